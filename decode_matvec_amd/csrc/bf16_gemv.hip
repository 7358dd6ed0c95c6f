// Plain BF16 GEMV, y = W x with fp32 accumulation: the uncompressed reference
// the fused compressed matvec is measured against on the same machine (no
// decode; not part of the method).
//
// Design for MI355X: one wave per row; each lane streams 16-byte chunks c =
// lane, lane + 64, ... of its row and of x, U chunks per loop trip, all loads
// of a trip issued before the first multiply, so a wave keeps U KiB of its row
// in flight and the grid (one wave per row, 4 rows per workgroup, far more
// workgroups than compute units) puts the whole matrix in flight as fast as
// the waves can issue.  The activations are read from the caches (every wave
// reads the same few KiB), never staged through LDS, so no barrier delays the
// first weight load.  Products of BF16 pairs accumulate in fp32 with
// v_dot2c_f32_bf16; a butterfly of lane shuffles sums the row.
//
// nwc_bf16_gemv_group runs several matrices in one launch (the same launch
// structure as nwc_matvec_group): what the first loads need (count, first
// workgroups, the weight pointers and row shapes of matrices 0..2) comes in
// the leading scalar arguments, which gfx950 preloads into scalar registers.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/nwc.h"

namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row
constexpr int kU = 8;             // 16-byte chunks per lane per loop trip

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x), acc,
                                         false);
}

// Sum of row `wr` (kc chunks of 8 BF16) against x; every lane of the wave
// returns the row sum.
// Weight loads are non-temporal like the compressed kernels' blob loads
// (each weight is read once per call).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4 *p) {
  const u32x4_nt v = __builtin_nontemporal_load((const u32x4_nt *)p);
  return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ float row_dot(const uint4 *__restrict__ wr, const uint4 *__restrict__ x, uint32_t kc,
                                         uint32_t lane) {
  float a0 = 0.f, a1 = 0.f;
  for (uint32_t c0 = 0; c0 < kc; c0 += 64 * kU) {
    uint4 wv[kU], xv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t c = c0 + u * 64 + lane;
      wv[u] = c < kc ? ld_nt(wr + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t c = c0 + u * 64 + lane;
      xv[u] = c < kc ? x[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      a0 = dot2(wv[u].x, xv[u].x, a0);
      a1 = dot2(wv[u].y, xv[u].y, a1);
      a0 = dot2(wv[u].z, xv[u].z, a0);
      a1 = dot2(wv[u].w, xv[u].w, a1);
    }
  }
  float a = a0 + a1;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
  return a;
}

__global__ __launch_bounds__(64 * kRowsPerBlock) void bf16_gemv_kernel(const uint4 *__restrict__ w,
                                                                       const uint4 *__restrict__ x,
                                                                       float *__restrict__ y, uint32_t n, uint32_t kc,
                                                                       uint32_t ldc) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t row = blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= n) return;
  const float a = row_dot(w + (uint64_t)row * ldc, x, kc, lane);
  if (lane == 0) y[row] = a;
}

// Group launch.  head: count | from_tail << 4 | grid << 5; begins: first
// workgroup of matrix 1 | of matrix 2 << 16; shape_m: n_m | kc_m << 17 (rows
// of kc_m chunks, row pitch kc_m).  from_tail: a matrix's shape or a first
// workgroup does not fit the packed fields, and everything comes from the tail.
constexpr uint32_t kGemvPreloaded = 3;
struct GemvTail {
  uint32_t begin[NWC_GROUP_MAX + 1];
  uint32_t n[NWC_GROUP_MAX], kc[NWC_GROUP_MAX], ldc[NWC_GROUP_MAX];
  const uint4 *w[NWC_GROUP_MAX];
  const uint4 *x[NWC_GROUP_MAX];
  float *y[NWC_GROUP_MAX];
};

__global__ __launch_bounds__(64 * kRowsPerBlock) void bf16_gemv_group_kernel(uint32_t head, uint32_t begins,
                                                                             uint32_t shape0, uint32_t shape1,
                                                                             uint32_t shape2,
                                                                             const uint4 *__restrict__ w0,
                                                                             const uint4 *__restrict__ w1,
                                                                             const uint4 *__restrict__ w2,
                                                                             const GemvTail tail) {
  const uint32_t count = head & 15u, wg = blockIdx.x, lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t m, beg, n, kc, ldc;
  const uint4 *w;
  if (count <= kGemvPreloaded && !((head >> 4) & 1u)) {
    const uint32_t all = head >> 5;
    const uint32_t b1 = count > 1 ? begins & 0xFFFFu : all, b2 = count > 2 ? begins >> 16 : all;
    m = wg >= b2 ? 2u : wg >= b1 ? 1u : 0u;
    beg = m == 0 ? 0u : m == 1 ? b1 : b2;
    const uint32_t sh = m == 0 ? shape0 : m == 1 ? shape1 : shape2;
    n = sh & 0x1FFFFu;
    kc = sh >> 17;
    ldc = kc;
    w = m == 0 ? w0 : m == 1 ? w1 : w2;
  } else {
    m = 0;
    for (uint32_t i = 1; i < count; ++i)
      if (wg >= tail.begin[i]) m = i;
    beg = tail.begin[m];
    n = tail.n[m];
    kc = tail.kc[m];
    ldc = tail.ldc[m];
    w = tail.w[m];
  }
  const uint32_t row = (wg - beg) * kRowsPerBlock + wave;
  if (row >= n) return;
  const float a = row_dot(w + (uint64_t)row * ldc, tail.x[m], kc, lane);
  if (lane == 0) tail.y[m][row] = a;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

int check_one(const void *d_w, int64_t n, int64_t k, int64_t ldw, const void *d_x, const float *d_y) {
  if (!d_w || !d_x || !d_y) return NWC_ERR_ARG;
  if (!aligned16(d_w) || !aligned16(d_x) || ((uintptr_t)d_y & 3)) return NWC_ERR_ARG;
  if (n < 1 || k < 8 || k % 8 || ldw < k || ldw % 8 || n >= ((int64_t)1 << 31) || ldw >= ((int64_t)1 << 34))
    return NWC_ERR_SHAPE;
  return NWC_OK;
}

}  // namespace

extern "C" int nwc_bf16_gemv(const void *d_w, int64_t n, int64_t k, int64_t ldw, const void *d_x, float *d_y,
                             void *stream) {
  const int st = check_one(d_w, n, k, ldw, d_x, d_y);
  if (st != NWC_OK) return st;
  const uint32_t blocks = (uint32_t)((n + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(bf16_gemv_kernel, dim3(blocks), dim3(64 * kRowsPerBlock), 0, (hipStream_t)stream,
                     (const uint4 *)d_w, (const uint4 *)d_x, d_y, (uint32_t)n, (uint32_t)(k / 8), (uint32_t)(ldw / 8));
  return hipGetLastError() == hipSuccess ? NWC_OK : NWC_ERR_HIP;
}

extern "C" int nwc_bf16_gemv_group(const nwc_bf16_gemv_desc *mats, int count, void *stream) {
  if (count < 0 || count > NWC_GROUP_MAX) return NWC_ERR_SHAPE;
  if (count == 0) return NWC_OK;
  if (!mats) return NWC_ERR_ARG;
  GemvTail tail;
  memset(&tail, 0, sizeof tail);
  uint64_t grid = 0;
  bool packable = count <= (int)kGemvPreloaded;
  uint32_t shape[3] = {0, 0, 0};
  for (int m = 0; m < count; ++m) {
    const nwc_bf16_gemv_desc &d = mats[m];
    const int st = check_one(d.d_w, d.n, d.k, d.ldw, d.d_x, d.d_y);
    if (st != NWC_OK) return st;
    tail.begin[m] = (uint32_t)grid;
    tail.n[m] = (uint32_t)d.n;
    tail.kc[m] = (uint32_t)(d.k / 8);
    tail.ldc[m] = (uint32_t)(d.ldw / 8);
    tail.w[m] = (const uint4 *)d.d_w;
    tail.x[m] = (const uint4 *)d.d_x;
    tail.y[m] = d.d_y;
    if (m < 3) {
      if (d.n >= (1 << 17) || d.k / 8 >= (1 << 15) || d.ldw != d.k) packable = false;
      shape[m] = (uint32_t)d.n | ((uint32_t)(d.k / 8) << 17);
    }
    grid += (uint64_t)((d.n + kRowsPerBlock - 1) / kRowsPerBlock);
  }
  if (grid >= ((uint64_t)1 << 31)) return NWC_ERR_SHAPE;
  tail.begin[count] = (uint32_t)grid;
  if (grid >= (1u << 27) || (count > 1 && tail.begin[1] > 0xFFFFu) || (count > 2 && tail.begin[2] > 0xFFFFu))
    packable = false;
  const uint32_t head = (uint32_t)count | (packable ? 0u : 1u << 4) | (packable ? (uint32_t)grid << 5 : 0u);
  const uint32_t begins = packable ? (count > 1 ? tail.begin[1] : 0u) | ((count > 2 ? tail.begin[2] : 0u) << 16) : 0u;
  hipLaunchKernelGGL(bf16_gemv_group_kernel, dim3((unsigned)grid), dim3(64 * kRowsPerBlock), 0, (hipStream_t)stream,
                     head, begins, shape[0], shape[1], shape[2], tail.w[0], count > 1 ? tail.w[1] : tail.w[0],
                     count > 2 ? tail.w[2] : tail.w[0], tail);
  return hipGetLastError() == hipSuccess ? NWC_OK : NWC_ERR_HIP;
}
