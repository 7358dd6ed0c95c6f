// gfx950 kernels of libnwc: fused decode + matvec, dequantization, gather.
//
// What is computed follows the "neural-weight-compression 0.9.0" PyPI page
// ("How it works": weights decoded in registers inside the matvec, fp32 row
// sums, dequantization and embedding lookup on the same decoder) and the
// "Qwen3-4B-NWC-fp8" model card (scale applied after the row sum).  The
// kernel design is this library's own, for CDNA4 wave64:
//
//  * One wave = one work item = 64 matrix rows x up to 256 columns.  Lane L
//    owns row L, so the activation pair of a step is the same for every lane
//    and lives in scalar registers; each lane keeps its own fp32 row sum and
//    no cross-lane reduction is needed inside an item.
//  * The item's code streams are staged once into LDS with coalesced 16-byte
//    loads, lane L's stream in LDS column L (bank L mod 32: conflict-free).
//  * Each step a lane reads 64 bits of its stream at its own bit position
//    (ds_read2st64), cuts a 12-bit peek with v_alignbit, and looks it up in a
//    16 KiB LDS table that yields the two exponent/sign bytes of the next two
//    weights (BF16) or one whole value (fp8) plus the bits consumed.  v_perm
//    joins them with the raw mantissa bytes into a BF16 pair and
//    v_dot2c_f32_bf16 accumulates it in fp32.  Peeks the table cannot finish
//    (escapes, long pairs) take a wave-uniform branch to an exact decoder.
//  * Raw mantissa bytes stream from HBM with 16-byte per-lane loads laid out
//    so a wave's load is one contiguous 1 KiB, prefetched four chunks ahead.
//  * Column spans of one row block are summed by the last wave to finish
//    (deterministic order, counters reset by that wave): one launch per matvec.
#include <hip/hip_runtime.h>

#include "nwc_check.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr uint32_t kSelLo = 0x05010400u;  // {m[0], hiA, m[1], hiB}
constexpr uint32_t kSelHi = 0x05030402u;  // {m[2], hiA, m[3], hiB}
constexpr uint32_t kSelPair = 0x05040100u; // {a.b0, a.b1, b.b0, b.b1}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct Geom {
  const uint8_t *blob;
  int64_t n, k;
  uint32_t cols, n_kspans, n_items, last_cols, k_pad, region_words;
  uint32_t r2s_lo, r2s_hi;  // rank_to_sym[0..7], one byte each
  uint64_t off_lut, off_items, off_mant, off_code;
};

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x), acc,
                                         false);
}

__device__ __forceinline__ uint32_t rank_sym(uint32_t r, uint32_t lo, uint32_t hi) {
  return ((r < 4 ? lo : hi) >> ((r & 3) * 8)) & 0x7Fu;
}

// 64 stream bits of this lane starting at bit P (valid: at least 33).
__device__ __forceinline__ uint64_t window64(const uint8_t *region, uint32_t lane4, uint32_t P) {
  const uint32_t a = ((P >> 5) << 8) + lane4;
  const uint32_t w0 = *(const uint32_t *)(region + a);
  const uint32_t w1 = *(const uint32_t *)(region + a + 256);
  return ((((uint64_t)w1) << 32) | w0) >> (P & 31);
}

// Exact decode of one BF16 code from the low bits of v: high byte and length.
__device__ __forceinline__ void bf16_code(uint32_t v, uint32_t lo, uint32_t hi, uint32_t &hb, uint32_t &len) {
  const uint32_t r = __builtin_ctz(~v | 0x100u);  // run of ones, capped at 8
  if (r < NWC_ESCAPE_R) {
    hb = (((v >> (r + 1)) & 1u) << 7) | rank_sym(r, lo, hi);
    len = r + 2;
  } else {
    hb = (((v >> 8) & 1u) << 7) | ((v >> 9) & 0x7Fu);
    len = 16;
  }
}

// Two BF16 codes at bit Q+2 in the table's entry format (slow path).
__device__ __noinline__ uint32_t bf16_pair_exact(const uint8_t *region, uint32_t lane4, uint32_t Q, uint32_t lo,
                                                 uint32_t hi) {
  const uint64_t v = window64(region, lane4, Q + NWC_LEAD_BITS);
  uint32_t ha, la, hb, lb;
  bf16_code((uint32_t)v, lo, hi, ha, la);
  bf16_code((uint32_t)(v >> la), lo, hi, hb, lb);
  return ha | (hb << 8) | ((la + lb) << 16);
}

__device__ __forceinline__ uint32_t fp8_to_bf16(uint32_t b) {
  const uint32_t s = (b >> 7) & 1u, E = (b >> 3) & 15u, M = b & 7u;
  if (E == 15u && M == 7u) return (s << 15) | 0x7FC0u;
  if (E == 0u) {
    if (M == 0u) return s << 15;
    const uint32_t p = 31u - __builtin_clz(M);
    return (s << 15) | ((p + 118u) << 7) | ((M ^ (1u << p)) << (7u - p));
  }
  return (s << 15) | ((E + 120u) << 7) | (M << 4);
}

// One fp8 code at bit Q+2 in the table's entry format (slow path).
__device__ __noinline__ uint32_t fp8_exact(const uint8_t *region, uint32_t lane4, uint32_t Q, uint32_t lo,
                                           uint32_t hi) {
  const uint32_t v = (uint32_t)window64(region, lane4, Q + NWC_LEAD_BITS);
  const uint32_t r = __builtin_ctz(~v | 0x100u);
  uint32_t s, E, M, len;
  if (r < NWC_ESCAPE_R) {
    s = (v >> (r + 1)) & 1u;
    M = (v >> (r + 2)) & 7u;
    E = rank_sym(r, lo, hi) & 15u;
    len = r + 5;
  } else {
    s = (v >> 8) & 1u;
    E = (v >> 9) & 15u;
    M = (v >> 13) & 7u;
    len = 16;
  }
  const uint32_t b = (s << 7) | (E << 3) | M;
  return fp8_to_bf16(b) | (b << 16) | (len << 24);
}

struct Lane {
  const uint8_t *region;  // this wave's staged code rows (LDS)
  const uint8_t *lut;     // decode table (LDS)
  uint32_t lane4;         // byte offset of this lane's column
  uint32_t Q;             // stream bit position of the next code, minus 2
  uint32_t lo, hi;        // rank_to_sym[0..7]
};

// Next two BF16 codes: returns {hiA, hiB, bits} entry.
__device__ __forceinline__ uint32_t bf16_step(Lane &s) {
  const uint32_t a = (__builtin_amdgcn_ubfe(s.Q, 5, 27) << 8) + s.lane4;  // row Q/32, column lane
  const uint32_t w0 = *(const uint32_t *)(s.region + a);
  const uint32_t w1 = *(const uint32_t *)(s.region + a + 256);
  const uint32_t W = __builtin_amdgcn_alignbit(w1, w0, s.Q);  // bits Q..Q+31; peek = bits 2..13
  uint32_t e = *(const uint32_t *)(s.lut + (W & 0x3FFCu));
  if (__builtin_expect(__any((int)e < 0), 0)) e = bf16_pair_exact(s.region, s.lane4, s.Q, s.lo, s.hi);
  s.Q += (e >> 16) & 0xFFu;
  return e;
}

// Next fp8 code: returns {bf16 value, byte, bits} entry.
__device__ __forceinline__ uint32_t fp8_step(Lane &s) {
  const uint32_t a = (__builtin_amdgcn_ubfe(s.Q, 5, 27) << 8) + s.lane4;  // row Q/32, column lane
  const uint32_t w0 = *(const uint32_t *)(s.region + a);
  const uint32_t w1 = *(const uint32_t *)(s.region + a + 256);
  const uint32_t W = __builtin_amdgcn_alignbit(w1, w0, s.Q);
  uint32_t e = *(const uint32_t *)(s.lut + (W & 0x3FFCu));
  if (__builtin_expect(__any((int)e < 0), 0)) e = fp8_exact(s.region, s.lane4, s.Q, s.lo, s.hi);
  s.Q += e >> 24;
  return e;
}

struct Item {
  uint32_t rb, ks, c0, ncols;
  int64_t row;
};

__device__ __forceinline__ Item item_of(const Geom &g, uint32_t item, uint32_t lane) {
  Item it;
  it.rb = item / g.n_kspans;
  it.ks = item - it.rb * g.n_kspans;
  it.c0 = it.ks * g.cols;
  it.ncols = it.ks == g.n_kspans - 1 ? g.last_cols : g.cols;
  it.row = (int64_t)it.rb * 64 + lane;
  return it;
}

// Copies the 16 KiB table into LDS (whole workgroup).
__device__ __forceinline__ void load_lut(const Geom &g, uint32_t *smem) {
  const uint4 *src = (const uint4 *)(g.blob + g.off_lut);
  uint4 *dst = (uint4 *)smem;
#pragma unroll
  for (int i = 0; i < NWC_LUT_BYTES / 16 / kThreads; ++i) dst[threadIdx.x + i * kThreads] = src[threadIdx.x + i * kThreads];
}

// Copies one item's code rows into the wave's LDS region (same layout).
__device__ __forceinline__ void stage_item(const Geom &g, uint32_t item, uint32_t lane, uint8_t *region) {
  const uint32_t *it = (const uint32_t *)(g.blob + g.off_items) + 2 * item;
  const uint32_t off = it[0], rows = it[1];
  const uint4 *src = (const uint4 *)(g.blob + g.off_code + off);
  uint4 *dst = (uint4 *)region;
  for (uint32_t i = lane; i < rows * 16; i += 64) dst[i] = src[i];
}

__device__ __forceinline__ const uint4 *mant_base(const Geom &g, const Item &it, uint32_t lane) {
  return (const uint4 *)(g.blob + g.off_mant + (uint64_t)it.rb * 64 * g.k_pad + (uint64_t)64 * it.c0) + lane;
}

// Activation pairs of 16 columns starting at item column `col` (zero past ncols).
__device__ __forceinline__ void x_pairs(const uint16_t *x, const Item &it, uint32_t col, bool full, uint32_t xs[8]) {
  if (full) {
    const uint32_t *x32 = (const uint32_t *)(x + it.c0 + col);
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[j] = x32[j];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t c = col + 2 * j;
      const uint32_t a = c < it.ncols ? x[it.c0 + c] : 0u;
      const uint32_t b = c + 1 < it.ncols ? x[it.c0 + c + 1] : 0u;
      xs[j] = a | (b << 16);
    }
  }
}

// ----------------------------------------------------------------- matvec
__device__ __forceinline__ void mv_group_bf16(Lane &s, const uint4 &m, const uint32_t xs[8], float &a0, float &a1) {
  const uint32_t mw[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t e = bf16_step(s);
    const uint32_t p = __builtin_amdgcn_perm(e, mw[j >> 1], (j & 1) ? kSelHi : kSelLo);
    if (j & 1)
      a1 = dot2(p, xs[j], a1);
    else
      a0 = dot2(p, xs[j], a0);
  }
}

__device__ __forceinline__ void mv_tail_bf16(Lane &s, const uint4 &m, const uint32_t xs[8], uint32_t left, float &a0,
                                             float &a1) {
  const uint32_t mw[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (2u * j >= left) break;
    const uint32_t e = bf16_step(s);
    uint32_t p = __builtin_amdgcn_perm(e, mw[j >> 1], (j & 1) ? kSelHi : kSelLo);
    if (2u * j + 1 >= left) p &= 0xFFFFu;  // column past the matrix edge: not a weight
    if (j & 1)
      a1 = dot2(p, xs[j], a1);
    else
      a0 = dot2(p, xs[j], a0);
  }
}

__device__ __forceinline__ void mv_group_fp8(Lane &s, const uint32_t xs[8], uint32_t left, float &a0, float &a1) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (2u * j >= left) break;
    const uint32_t ea = fp8_step(s);
    uint32_t eb = 0;
    if (2u * j + 1 < left) eb = fp8_step(s);
    const uint32_t p = __builtin_amdgcn_perm(eb, ea, kSelPair);
    if (j & 1)
      a1 = dot2(p, xs[j], a1);
    else
      a0 = dot2(p, xs[j], a0);
  }
}

// Row sum of one item for this lane.
template <bool FP8>
__device__ __forceinline__ float item_rowsum(const Geom &g, const Item &it, Lane &s, const uint16_t *x, uint32_t lane) {
  float a0 = 0.f, a1 = 0.f;
  const uint32_t nfull = it.ncols >> 4, left = it.ncols & 15u;
  uint32_t xs[8];
  if (!FP8) {
    const uint4 *mp = mant_base(g, it, lane);
    const uint4 zero = {0u, 0u, 0u, 0u};
    uint4 mt = left ? mp[nfull * 64] : zero;
    uint4 m0 = nfull > 0 ? mp[0] : zero, m1 = nfull > 1 ? mp[64] : zero;
    uint4 m2 = nfull > 2 ? mp[128] : zero, m3 = nfull > 3 ? mp[192] : zero;
    for (uint32_t g0 = 0; g0 < nfull; g0 += 4) {
      x_pairs(x, it, g0 * 16, true, xs);
      mv_group_bf16(s, m0, xs, a0, a1);
      if (g0 + 4 < nfull) m0 = mp[(g0 + 4) * 64];
      if (g0 + 1 < nfull) {
        x_pairs(x, it, (g0 + 1) * 16, true, xs);
        mv_group_bf16(s, m1, xs, a0, a1);
        if (g0 + 5 < nfull) m1 = mp[(g0 + 5) * 64];
      }
      if (g0 + 2 < nfull) {
        x_pairs(x, it, (g0 + 2) * 16, true, xs);
        mv_group_bf16(s, m2, xs, a0, a1);
        if (g0 + 6 < nfull) m2 = mp[(g0 + 6) * 64];
      }
      if (g0 + 3 < nfull) {
        x_pairs(x, it, (g0 + 3) * 16, true, xs);
        mv_group_bf16(s, m3, xs, a0, a1);
        if (g0 + 7 < nfull) m3 = mp[(g0 + 7) * 64];
      }
    }
    if (left) {
      x_pairs(x, it, nfull * 16, false, xs);
      mv_tail_bf16(s, mt, xs, left, a0, a1);
    }
  } else {
    for (uint32_t gi = 0; gi < nfull; ++gi) {
      x_pairs(x, it, gi * 16, true, xs);
      mv_group_fp8(s, xs, 16, a0, a1);
    }
    if (left) {
      x_pairs(x, it, nfull * 16, false, xs);
      mv_group_fp8(s, xs, left, a0, a1);
    }
  }
  return a0 + a1;
}

template <bool FP8>
__global__ __launch_bounds__(kThreads) void matvec_kernel(Geom g, const uint16_t *__restrict__ x,
                                                          const float *__restrict__ scale, float *__restrict__ y,
                                                          float *__restrict__ partial, uint32_t *__restrict__ count) {
  __shared__ uint32_t s_lut[NWC_LUT_ENTRIES];
  extern __shared__ uint32_t s_code[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t item = blockIdx.x * kWaves + wave;
  uint8_t *region = (uint8_t *)(s_code + wave * g.region_words);
  load_lut(g, s_lut);
  const bool active = item < g.n_items;
  if (active) stage_item(g, item, lane, region);
  __syncthreads();
  if (!active) return;

  const Item it = item_of(g, item, lane);
  Lane s{region, (const uint8_t *)s_lut, lane * 4u, 0u, g.r2s_lo, g.r2s_hi};
  float acc = item_rowsum<FP8>(g, it, s, x, lane);

  if (g.n_kspans == 1) {
    if (it.row < g.n) y[it.row] = FP8 ? acc * scale[it.row] : acc;
    return;
  }
  __hip_atomic_store(partial + (uint64_t)item * 64 + lane, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __threadfence();
  uint32_t done = 0;
  if (lane == 0) done = atomicAdd(count + it.rb, 1u);
  done = __builtin_amdgcn_readfirstlane(done);
  if (done != g.n_kspans - 1) return;
  __threadfence();
  float sum = 0.f;
  const float *p = partial + (uint64_t)it.rb * g.n_kspans * 64 + lane;
  for (uint32_t j = 0; j < g.n_kspans; ++j)
    sum += __hip_atomic_load(p + (uint64_t)j * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (it.row < g.n) y[it.row] = FP8 ? sum * scale[it.row] : sum;
  if (lane == 0) __hip_atomic_store(count + it.rb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------- dequant / gather
// Decodes the lane's item stream and hands each BF16 pair (or fp8 byte) to out.
template <bool FP8, class Out>
__device__ __forceinline__ void item_decode(const Geom &g, const Item &it, Lane &s, const uint4 *mp, Out &out) {
  const uint32_t nsteps = FP8 ? it.ncols : (it.ncols + 1) / 2;
  for (uint32_t gi = 0; gi * 16 < it.ncols; ++gi) {
    uint32_t mw[4] = {0u, 0u, 0u, 0u};
    if (!FP8) {
      const uint4 m = mp[gi * 64];
      mw[0] = m.x; mw[1] = m.y; mw[2] = m.z; mw[3] = m.w;
    }
    const uint32_t per = FP8 ? 16u : 8u;
#pragma unroll
    for (uint32_t j = 0; j < per; ++j) {
      const uint32_t t = gi * per + j;
      if (t >= nsteps) break;
      if (FP8) {
        const uint32_t e = fp8_step(s);
        out.put8(gi * 16 + j, (e >> 16) & 0xFFu);
      } else {
        const uint32_t e = bf16_step(s);
        out.put16(gi * 16 + 2 * j, __builtin_amdgcn_perm(e, mw[j >> 1], (j & 1) ? kSelHi : kSelLo));
      }
    }
  }
}

// Writes one row segment; pairs for columns past ncols are dropped.
struct RowOut {
  uint8_t *dst;    // element (row, c0)
  uint32_t ncols;
  bool ok;
  __device__ __forceinline__ void put16(uint32_t c, uint32_t pair) {
    if (!ok) return;
    uint16_t *d = (uint16_t *)dst;
    d[c] = (uint16_t)pair;
    if (c + 1 < ncols) d[c + 1] = (uint16_t)(pair >> 16);
  }
  __device__ __forceinline__ void put8(uint32_t c, uint32_t b) {
    if (ok) dst[c] = (uint8_t)b;
  }
};

template <bool FP8>
__global__ __launch_bounds__(kThreads) void dequant_kernel(Geom g, uint8_t *__restrict__ w, int64_t ld) {
  __shared__ uint32_t s_lut[NWC_LUT_ENTRIES];
  extern __shared__ uint32_t s_code[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t item = blockIdx.x * kWaves + wave;
  uint8_t *region = (uint8_t *)(s_code + wave * g.region_words);
  load_lut(g, s_lut);
  const bool active = item < g.n_items;
  if (active) stage_item(g, item, lane, region);
  __syncthreads();
  if (!active) return;
  const Item it = item_of(g, item, lane);
  Lane s{region, (const uint8_t *)s_lut, lane * 4u, 0u, g.r2s_lo, g.r2s_hi};
  const int64_t esz = FP8 ? 1 : 2;
  RowOut out{w + (it.row * ld + it.c0) * esz, it.ncols, it.row < g.n};
  item_decode<FP8>(g, it, s, FP8 ? nullptr : mant_base(g, it, lane), out);
}

template <bool FP8>
__global__ __launch_bounds__(kThreads) void gather_kernel(Geom g, const int64_t *__restrict__ ids, int64_t n_ids,
                                                          uint8_t *__restrict__ out) {
  __shared__ uint32_t s_lut[NWC_LUT_ENTRIES];
  extern __shared__ uint32_t s_code[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t *region = (uint8_t *)(s_code + wave * g.region_words);
  load_lut(g, s_lut);
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool live = t < n_ids;
  const int64_t id = live ? ids[t] : 0;
  const bool valid = live && id >= 0 && id < g.n;
  const int64_t row = valid ? id : 0;
  const uint32_t rb = (uint32_t)(row >> 6), L = (uint32_t)(row & 63);
  const int64_t esz = FP8 ? 1 : 2;
  for (uint32_t ks = 0; ks < g.n_kspans; ++ks) {
    const uint32_t item = rb * g.n_kspans + ks;
    const uint32_t *ie = (const uint32_t *)(g.blob + g.off_items) + 2 * item;
    const uint32_t off = ie[0], rows = ie[1];
    const uint32_t *src = (const uint32_t *)(g.blob + g.off_code + off) + L;
    uint32_t *dst = (uint32_t *)region + lane;
    for (uint32_t r = 0; r < rows; ++r) dst[r * 64] = src[r * 64];
    Item it;
    it.rb = rb;
    it.ks = ks;
    it.c0 = ks * g.cols;
    it.ncols = ks == g.n_kspans - 1 ? g.last_cols : g.cols;
    it.row = row;
    Lane s{region, (const uint8_t *)s_lut, lane * 4u, 0u, g.r2s_lo, g.r2s_hi};
    RowOut o{out + (t * g.k + it.c0) * esz, it.ncols, live};
    const uint4 *mp = FP8 ? nullptr : mant_base(g, it, L);
    if (valid) {
      item_decode<FP8>(g, it, s, mp, o);
    } else if (live) {
      for (uint32_t c = 0; c < it.ncols * esz; ++c) o.dst[c] = 0;
    }
  }
}

Geom make_geom(const nwc_header_t &h, const void *d_blob) {
  Geom g;
  g.blob = (const uint8_t *)d_blob;
  g.n = h.n;
  g.k = h.k;
  g.cols = h.cols_per_item;
  g.n_kspans = h.n_kspans;
  g.n_items = h.n_items;
  g.last_cols = h.last_cols;
  g.k_pad = h.k_pad;
  g.region_words = (h.max_rows + NWC_GUARD_ROWS) * 64;
  g.r2s_lo = h.rank_to_sym[0] | (h.rank_to_sym[1] << 8) | (h.rank_to_sym[2] << 16) | ((uint32_t)h.rank_to_sym[3] << 24);
  g.r2s_hi = h.rank_to_sym[4] | (h.rank_to_sym[5] << 8) | (h.rank_to_sym[6] << 16) | ((uint32_t)h.rank_to_sym[7] << 24);
  g.off_lut = h.off_lut;
  g.off_items = h.off_items;
  g.off_mant = h.off_mant;
  g.off_code = h.off_code;
  return g;
}

// Dynamic LDS: the waves' code regions (the decode table is static LDS).
size_t lds_bytes(const Geom &g) { return (size_t)kWaves * g.region_words * 4; }

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int launched() { return hipGetLastError() == hipSuccess ? NWC_OK : NWC_ERR_HIP; }

int read_header(const void *header, nwc_header_t &h) {
  if (!header) return NWC_ERR_ARG;
  memcpy(&h, header, sizeof h);
  return nwc_check_header(&h);
}

}  // namespace

extern "C" {

int nwc_matvec(const void *header, const void *d_blob, const void *d_x, const float *d_scale, float *d_y, void *d_ws,
               int64_t ws_bytes, void *stream) {
  nwc_header_t h;
  int st = read_header(header, h);
  if (st != NWC_OK) return st;
  if (!d_blob || !d_x || !d_y || !aligned(d_blob, 16) || !aligned(d_x, 16) || !aligned(d_y, 4)) return NWC_ERR_ARG;
  const bool fp8 = h.elem == NWC_FP8_E4M3;
  if (fp8 != (d_scale != nullptr) || (d_scale && !aligned(d_scale, 4))) return NWC_ERR_ARG;
  int64_t need = 0;
  if ((st = nwc_workspace_size(header, &need)) != NWC_OK) return st;
  float *partial = nullptr;
  uint32_t *count = nullptr;
  if (need > 0) {
    if (!d_ws || !aligned(d_ws, 256)) return NWC_ERR_ARG;
    if (ws_bytes < need) return NWC_ERR_CAPACITY;
    partial = (float *)d_ws;
    count = (uint32_t *)((uint8_t *)d_ws + nwc_round_up((int64_t)h.n_items * 64 * 4, 256));
  }
  const Geom g = make_geom(h, d_blob);
  const dim3 grid((h.n_items + kWaves - 1) / kWaves), block(kThreads);
  hipStream_t s = (hipStream_t)stream;
  if (fp8)
    hipLaunchKernelGGL(matvec_kernel<true>, grid, block, lds_bytes(g), s, g, (const uint16_t *)d_x, d_scale, d_y,
                       partial, count);
  else
    hipLaunchKernelGGL(matvec_kernel<false>, grid, block, lds_bytes(g), s, g, (const uint16_t *)d_x, d_scale, d_y,
                       partial, count);
  return launched();
}

int nwc_dequant(const void *header, const void *d_blob, void *d_w, int64_t ld, void *stream) {
  nwc_header_t h;
  int st = read_header(header, h);
  if (st != NWC_OK) return st;
  if (!d_blob || !d_w || !aligned(d_blob, 16) || !aligned(d_w, 16)) return NWC_ERR_ARG;
  if (ld < h.k) return NWC_ERR_SHAPE;
  const Geom g = make_geom(h, d_blob);
  const dim3 grid((h.n_items + kWaves - 1) / kWaves), block(kThreads);
  hipStream_t s = (hipStream_t)stream;
  if (h.elem == NWC_FP8_E4M3)
    hipLaunchKernelGGL(dequant_kernel<true>, grid, block, lds_bytes(g), s, g, (uint8_t *)d_w, ld);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, grid, block, lds_bytes(g), s, g, (uint8_t *)d_w, ld);
  return launched();
}

int nwc_gather(const void *header, const void *d_blob, const int64_t *d_ids, int64_t n_ids, void *d_out,
               void *stream) {
  nwc_header_t h;
  int st = read_header(header, h);
  if (st != NWC_OK) return st;
  if (n_ids < 0 || n_ids > ((int64_t)1 << 31)) return NWC_ERR_SHAPE;
  if (n_ids == 0) return NWC_OK;
  if (!d_blob || !d_ids || !d_out || !aligned(d_blob, 16) || !aligned(d_ids, 8) || !aligned(d_out, 16))
    return NWC_ERR_ARG;
  const Geom g = make_geom(h, d_blob);
  const dim3 grid((unsigned)((n_ids + kThreads - 1) / kThreads)), block(kThreads);
  hipStream_t s = (hipStream_t)stream;
  if (h.elem == NWC_FP8_E4M3)
    hipLaunchKernelGGL(gather_kernel<true>, grid, block, lds_bytes(g), s, g, d_ids, n_ids, (uint8_t *)d_out);
  else
    hipLaunchKernelGGL(gather_kernel<false>, grid, block, lds_bytes(g), s, g, d_ids, n_ids, (uint8_t *)d_out);
  return launched();
}

}  // extern "C"
