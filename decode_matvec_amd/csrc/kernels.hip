// gfx950 kernels of libnwc: fused decode + matvec, dequantization, gather.
//
// What is computed follows the "neural-weight-compression 0.9.0" PyPI page
// ("How it works": weights decoded in registers inside the matvec, fp32 row
// sums, dequantization and embedding lookup on the same decoder) and the
// "Qwen3-4B-NWC-fp8" model card (scale applied after the row sum).  The
// kernel design is this library's own, for CDNA4 wave64:
//
//  * A work item is 64 matrix rows x up to 256 columns; lane L owns row L, so
//    the activation pair of a decode step is the same for every lane and no
//    cross-lane reduction is needed inside an item.
//  * A wave decodes NI items of consecutive row blocks at the same column span
//    side by side (NI independent decode chains per lane), which hides LDS
//    latency and shares the activation loads.
//  * Each item's code streams are staged once into LDS with coalesced 16-byte
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
//  * Each wave stores its item's 64 row sums as plain fp32 partials; when a
//    matrix has more than one column span, a second small kernel sums each
//    row's partials in a fixed order (deterministic, no atomics, no fences).
#include <hip/hip_runtime.h>

#include "nwc_check.h"

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr uint32_t kSelLo = 0x05010400u;   // {m[0], hiA, m[1], hiB}
constexpr uint32_t kSelHi = 0x05030402u;   // {m[2], hiA, m[3], hiB}
constexpr uint32_t kSelPair = 0x05040100u; // {a.b0, a.b1, b.b0, b.b1}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint32_t lds_u32;

struct Geom {
  const uint8_t *blob;
  int64_t n, k;
  uint32_t cols, n_rowblocks, n_kspans, n_items, last_cols, k_pad, region_words;
  uint32_t r2s_lo, r2s_hi;  // rank_to_sym[0..7], one byte each
  uint64_t off_lut, off_items, off_mant, off_code;
};

// ----------------------------------------------------------------- LDS helpers
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(size_t)(const lds_u32 *)p;
}
__device__ __forceinline__ uint32_t lds_load(uint32_t byte_addr) { return *(const lds_u32 *)(size_t)byte_addr; }
// Byte address of stream word (Q / 32) in the lane column starting at col_base.
__device__ __forceinline__ uint32_t word_addr(uint32_t col_base, uint32_t Q) {
  uint32_t a;
  asm("v_lshl_add_u32 %0, %1, 8, %2" : "=v"(a) : "v"(Q >> 5), "v"(col_base));
  return a;
}

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x), acc,
                                         false);
}

__device__ __forceinline__ uint32_t rank_sym(uint32_t r, uint32_t lo, uint32_t hi) {
  return ((r < 4 ? lo : hi) >> ((r & 3) * 8)) & 0x7Fu;
}

// 64 stream bits of a lane starting at bit P (at least 33 of them valid).
__device__ __forceinline__ uint64_t window64(uint32_t col_base, uint32_t P) {
  const uint32_t a = word_addr(col_base, P);
  const uint32_t w0 = lds_load(a), w1 = lds_load(a + 256);
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

// Two BF16 codes at bit Q+2, in the decode table's entry format (slow path).
__device__ __noinline__ uint32_t bf16_pair_exact(uint32_t col_base, uint32_t Q, uint32_t lo, uint32_t hi) {
  const uint64_t v = window64(col_base, Q + NWC_LEAD_BITS);
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

// One fp8 code at bit Q+2, in the decode table's entry format (slow path).
__device__ __noinline__ uint32_t fp8_exact(uint32_t col_base, uint32_t Q, uint32_t lo, uint32_t hi) {
  const uint32_t v = (uint32_t)window64(col_base, Q + NWC_LEAD_BITS);
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

// Decode state of one stream.
struct Lane {
  uint32_t col;  // LDS byte address of this lane's column (region + 4*lane)
  uint32_t lut;  // LDS byte address of the decode table
  uint32_t Q;    // stream bit position of the next code, minus 2
  uint32_t lo, hi;
};

// Next two BF16 codes of NI streams: e[i] = {hiA, hiB, bits} entries.
template <int NI>
__device__ __forceinline__ void bf16_steps(Lane (&s)[NI], uint32_t (&e)[NI]) {
  uint32_t w0[NI], w1[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t a = word_addr(s[i].col, s[i].Q);
    w0[i] = lds_load(a);
    w1[i] = lds_load(a + 256);
  }
  uint32_t any = 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t W = __builtin_amdgcn_alignbit(w1[i], w0[i], s[i].Q);  // bits Q..Q+31; peek = bits 2..13
    e[i] = lds_load(s[i].lut + (W & 0x3FFCu));
    any |= e[i];
  }
  if (__builtin_expect(__any((int)any < 0), 0)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) e[i] = bf16_pair_exact(s[i].col, s[i].Q, s[i].lo, s[i].hi);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) s[i].Q += (e[i] >> 16) & 0xFFu;
}

// Next fp8 code: returns {bf16 value, byte, bits}.
__device__ __forceinline__ uint32_t fp8_step(Lane &s) {
  const uint32_t a = word_addr(s.col, s.Q);
  const uint32_t W = __builtin_amdgcn_alignbit(lds_load(a + 256), lds_load(a), s.Q);
  uint32_t e = lds_load(s.lut + (W & 0x3FFCu));
  if (__builtin_expect(__any((int)e < 0), 0)) e = fp8_exact(s.col, s.Q, s.lo, s.hi);
  s.Q += e >> 24;
  return e;
}

__device__ __forceinline__ uint32_t bf16_step(Lane &s) {
  Lane one[1] = {s};
  uint32_t e[1];
  bf16_steps<1>(one, e);
  s = one[0];
  return e[0];
}

// Copies the 16 KiB decode table into LDS (whole workgroup).
__device__ __forceinline__ void load_lut(const Geom &g, uint32_t *lut) {
  const uint4 *src = (const uint4 *)(g.blob + g.off_lut);
  uint4 *dst = (uint4 *)lut;
#pragma unroll
  for (int i = 0; i < NWC_LUT_BYTES / 16 / kThreads; ++i)
    dst[threadIdx.x + i * kThreads] = src[threadIdx.x + i * kThreads];
}

// Copies one item's code rows into an LDS region (same layout).
__device__ __forceinline__ void stage_item(const Geom &g, uint32_t item, uint32_t lane, uint32_t *region) {
  const uint32_t *it = (const uint32_t *)(g.blob + g.off_items) + 2 * item;
  const uint32_t off = it[0], rows = it[1];
  const uint4 *src = (const uint4 *)(g.blob + g.off_code + off);
  uint4 *dst = (uint4 *)region;
  for (uint32_t i = lane; i < rows * 16; i += 64) dst[i] = src[i];
}

// Mantissa chunk 0 of this lane for item (rb, column c0); chunk j is at +64*j.
__device__ __forceinline__ const uint4 *mant_base(const Geom &g, uint32_t rb, uint32_t c0, uint32_t lane) {
  return (const uint4 *)(g.blob + g.off_mant + (uint64_t)rb * 64 * g.k_pad + (uint64_t)64 * c0) + lane;
}

// A VGPR holding 0 that the compiler cannot see through.  Added to a uniform
// address it keeps the load a vector load (vmcnt) rather than a scalar one,
// whose completion every LDS wait would also have to wait for (lgkmcnt).
__device__ __forceinline__ uint32_t opaque_zero() {
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// Activation pairs of 16 columns starting at absolute column c (all inside).
struct X8 {
  uint32_t v[8];
};
__device__ __forceinline__ X8 load_x8(const uint16_t *x, uint32_t c, uint32_t z) {
  const uint4 *p = (const uint4 *)(x + c) + z;
  const uint4 a = p[0], b = p[1];
  return X8{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}
// Same for the last, partial group: columns c .. c+left-1, zero beyond.
__device__ __forceinline__ X8 load_x8_tail(const uint16_t *x, uint32_t c, uint32_t left, uint32_t z) {
  X8 r;
#pragma unroll
  for (uint32_t j = 0; j < 8; ++j) {
    const uint32_t a = 2 * j < left ? x[c + 2 * j + z] : 0u;
    const uint32_t b = 2 * j + 1 < left ? x[c + 2 * j + 1 + z] : 0u;
    r.v[j] = a | (b << 16);
  }
  return r;
}

// ----------------------------------------------------------------- matvec
// One group (16 columns) of NI BF16 streams: 8 two-code steps each.
template <int NI>
__device__ __forceinline__ void mv_group_bf16(Lane (&s)[NI], const uint4 (&m)[NI], const X8 &x, float (&a0)[NI],
                                              float (&a1)[NI], uint32_t left) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (2u * j >= left) break;
    uint32_t e[NI];
    bf16_steps<NI>(s, e);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t mw = (j >> 1) == 0 ? m[i].x : (j >> 1) == 1 ? m[i].y : (j >> 1) == 2 ? m[i].z : m[i].w;
      uint32_t p = __builtin_amdgcn_perm(e[i], mw, (j & 1) ? kSelHi : kSelLo);
      if (2u * j + 1 >= left) p &= 0xFFFFu;  // column past the matrix edge: not a weight
      if (j & 1)
        a1[i] = dot2(p, x.v[j], a1[i]);
      else
        a0[i] = dot2(p, x.v[j], a0[i]);
    }
  }
}

// Loads a matvec item needs before its first step.  The mantissa chunks go
// through a ring of depth D: chunks 0..D-1 are requested in the prologue and
// chunk g+D while group g decodes, so an item's bytes are requested as its
// decode progresses rather than all at kernel start (with every wave of a
// matrix resident at once, the latter queues the whole matrix in HBM ahead of
// the first decode step).
template <int NI, int D>
struct MvPrefetch {
  const uint4 *mp[NI];  // this lane's mantissa chunk 0 per item
  uint4 m[D][NI];       // the ring
  X8 xc;                // activations of group 0
  uint32_t nfull, left, last, z;
};

// Issued after the item's direct-to-LDS copies: the activations of group 0
// (skipped for an item without a full group), then exactly D*NI mantissa
// chunk loads.  The kernel then waits with vmcnt(D*NI) -- for the copies and
// the activations only.  Chunk indices are clamped to one that exists (an
// item always has at least one 16-column chunk), so every load is
// unconditional and no merge of an in-flight load makes the compiler wait for
// all of them.
template <int NI, int D>
__device__ __forceinline__ void mv_prefetch(MvPrefetch<NI, D> &p, const Geom &g, const uint32_t (&rb)[NI],
                                            uint32_t c0, uint32_t ncols, const uint16_t *x, uint32_t lane) {
  p.nfull = ncols >> 4;
  p.left = ncols & 15u;
  p.last = p.nfull > 0 ? p.nfull - 1 : 0;
  p.z = opaque_zero();
  if (p.nfull > 0) p.xc = load_x8(x, c0, p.z);
#pragma unroll
  for (int i = 0; i < NI; ++i) p.mp[i] = mant_base(g, rb[i], c0, lane);
#pragma unroll
  for (int r = 0; r < D; ++r)
#pragma unroll
    for (int i = 0; i < NI; ++i) p.m[r][i] = p.mp[i][((uint32_t)r < p.last ? (uint32_t)r : p.last) * 64];
}

// Row sums of NI BF16 items (row blocks rb[i], same column span) for this lane.
template <int NI, int D>
__device__ __forceinline__ void mv_run(MvPrefetch<NI, D> &p, Lane (&s)[NI], uint32_t c0, const uint16_t *x,
                                       float (&out)[NI]) {
  float a0[NI], a1[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) a0[i] = a1[i] = 0.f;
  X8 xc = p.xc;
  for (uint32_t g0 = 0; g0 < p.nfull; g0 += D) {
#pragma unroll
    for (uint32_t r = 0; r < (uint32_t)D; ++r) {
      const uint32_t gi = g0 + r;
      if (gi >= p.nfull) break;
      const uint32_t gn = gi + 1 < p.last ? gi + 1 : p.last;
      const X8 xn = load_x8(x, c0 + gn * 16, p.z);
      mv_group_bf16<NI>(s, p.m[r], xc, a0, a1, 16);
      const uint32_t gf = gi + D < p.last ? gi + D : p.last;
#pragma unroll
      for (int i = 0; i < NI; ++i) p.m[r][i] = p.mp[i][gf * 64];
      xc = xn;
    }
  }
  if (p.left) {
    uint4 mt[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) mt[i] = p.mp[i][p.nfull * 64];
    const X8 xt = load_x8_tail(x, c0 + p.nfull * 16, p.left, p.z);
    mv_group_bf16<NI>(s, mt, xt, a0, a1, p.left);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) out[i] = a0[i] + a1[i];
}

// Row sum of one fp8 item for this lane (one code per step).
__device__ __forceinline__ float rowsum_fp8(uint32_t c0, uint32_t ncols, Lane &s, const uint16_t *x) {
  const uint32_t z = opaque_zero();
  float a0 = 0.f, a1 = 0.f;
  for (uint32_t col = 0; col < ncols; col += 16) {
    const uint32_t left = ncols - col < 16 ? ncols - col : 16;
    const X8 xv = left == 16 ? load_x8(x, c0 + col, z) : load_x8_tail(x, c0 + col, left, z);
#pragma unroll
    for (uint32_t j = 0; j < 8; ++j) {
      if (2 * j >= left) break;
      const uint32_t ea = fp8_step(s);
      const uint32_t eb = 2 * j + 1 < left ? fp8_step(s) : 0u;
      const uint32_t p = __builtin_amdgcn_perm(eb, ea, kSelPair);
      if (j & 1)
        a1 = dot2(p, xv.v[j], a1);
      else
        a0 = dot2(p, xv.v[j], a0);
    }
  }
  return a0 + a1;
}

// ----------------------------------------------------------------- async staging
typedef __attribute__((address_space(3))) void lds_void;

// This wave's share of a copy global -> LDS: 1 KiB per instruction straight
// into LDS (no registers), lane L moving bytes [16L, 16L+16) of each KiB.
__device__ __forceinline__ void dma_to_lds(const uint8_t *src, uint32_t *dst, uint32_t bytes, uint32_t lane) {
  for (uint32_t off = 0; off < bytes; off += 1024)
    if (off + lane * 16 < bytes)
      __builtin_amdgcn_global_load_lds(src + off + lane * 16, (lds_void *)((uint8_t *)dst + off), 16, 0, 0);
}

__device__ __forceinline__ void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Waits until at most N vector loads are outstanding: with N mantissa loads
// issued last, this waits for everything issued before them.
template <int N>
__device__ __forceinline__ void wait_copies_before(bool issued) {
  if (issued)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  else
    wait_all_loads();
}

// Partial sums live at [row][column span], each row padded to a multiple of
// 4 spans (16-byte loads in the reduction).
__device__ __forceinline__ uint32_t kspans_pad(uint32_t n_kspans) { return (n_kspans + 3u) & ~3u; }

// Wave w of the grid decodes row blocks NI*j .. NI*j+NI-1 at column span ks,
// where w = j * n_kspans + ks, and writes y (one span) or its partial sums.
template <bool FP8, int NI, int D>
__global__ __launch_bounds__(kThreads) void matvec_kernel(Geom g, const uint32_t *__restrict__ items,
                                                          const uint16_t *__restrict__ x,
                                                          const float *__restrict__ scale, float *__restrict__ y,
                                                          float *__restrict__ partial) {
  __shared__ uint32_t s_lut[NWC_LUT_ENTRIES];
  extern __shared__ uint32_t s_code[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t witem = blockIdx.x * kWaves + wave;
  const uint32_t n_groups = (g.n_rowblocks + NI - 1) / NI;
  const bool active = witem < n_groups * g.n_kspans;
  const uint32_t grp = active ? witem / g.n_kspans : 0, ks = active ? witem - grp * g.n_kspans : 0;
  const uint32_t c0 = ks * g.cols;
  const uint32_t ncols = ks == g.n_kspans - 1 ? g.last_cols : g.cols;

  // Issue everything the first step needs, then wait once.  The item table
  // entries are wave-uniform scalar loads, so waiting for them (lgkmcnt) does
  // not wait for the decode-table copy already in flight (vmcnt).
  uint32_t rb[NI], code_off[NI], code_rows[NI];
  uint32_t *region[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t r = grp * NI + i;
    rb[i] = r < g.n_rowblocks ? r : g.n_rowblocks - 1;
    region[i] = s_code + (wave * NI + i) * g.region_words;
    code_off[i] = items[2 * (rb[i] * g.n_kspans + ks)];
    code_rows[i] = items[2 * (rb[i] * g.n_kspans + ks) + 1];
  }
  dma_to_lds(g.blob + g.off_lut + wave * (NWC_LUT_BYTES / kWaves), s_lut + wave * (NWC_LUT_ENTRIES / kWaves),
             NWC_LUT_BYTES / kWaves, lane);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    if (active) dma_to_lds(g.blob + g.off_code + code_off[i], region[i], code_rows[i] * 256, lane);
  MvPrefetch<NI, D> pf;
  if (!FP8) {
    if (active) mv_prefetch<NI, D>(pf, g, rb, c0, ncols, x, lane);
    wait_copies_before<D * NI>(active);
  } else {
    wait_all_loads();
  }
  // Each wave has waited for its own copies into LDS; a bare barrier then
  // makes all of them visible.  (__syncthreads() would add a fence that waits
  // for every outstanding load, including the mantissa chunks meant to keep
  // streaming in during the first groups.)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (!active) return;

  const uint32_t lut = lds_addr(s_lut);
  float acc[NI];
  if (FP8) {
    Lane s{lds_addr(region[0]) + 4 * lane, lut, 0u, g.r2s_lo, g.r2s_hi};
    acc[0] = rowsum_fp8(c0, ncols, s, x);
  } else {
    Lane s[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) s[i] = Lane{lds_addr(region[i]) + 4 * lane, lut, 0u, g.r2s_lo, g.r2s_hi};
    mv_run<NI, D>(pf, s, c0, x, acc);
  }
  const uint32_t kp = kspans_pad(g.n_kspans);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (grp * NI + i >= g.n_rowblocks) continue;
    const int64_t row = (int64_t)rb[i] * 64 + lane;
    if (g.n_kspans == 1) {
      if (row < g.n) y[row] = FP8 ? acc[i] * scale[row] : acc[i];
    } else {
      partial[(uint64_t)row * kp + ks] = acc[i];
    }
  }
}

// y[row] = (scale[row] *) sum over column spans of the partials, 16 threads
// per row: thread j sums 16-byte chunks j, j+16, ... in order, then a fixed
// butterfly over the 16 threads.  Same order every call.
template <bool FP8>
__global__ __launch_bounds__(256) void reduce_kernel(const float *__restrict__ partial, uint32_t n_kspans, int64_t n,
                                                     const float *__restrict__ scale, float *__restrict__ y) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t >> 4;
  const uint32_t j = (uint32_t)t & 15u;
  const uint32_t kp = kspans_pad(n_kspans);
  float sum = 0.f;
  if (row < n) {
    const float4 *p = (const float4 *)(partial + (uint64_t)row * kp);
    for (uint32_t c = j; c < kp / 4; c += 16) {
      const float4 v = p[c];
      sum += v.x;
      if (4 * c + 1 < n_kspans) sum += v.y;
      if (4 * c + 2 < n_kspans) sum += v.z;
      if (4 * c + 3 < n_kspans) sum += v.w;
    }
  }
  sum += __shfl_xor(sum, 8, 16);
  sum += __shfl_xor(sum, 4, 16);
  sum += __shfl_xor(sum, 2, 16);
  sum += __shfl_xor(sum, 1, 16);
  if (j == 0 && row < n) y[row] = FP8 ? sum * scale[row] : sum;
}

// ----------------------------------------------------------------- dequant / gather
// Decodes the lane's item stream and hands each BF16 pair (or fp8 byte) to out.
template <bool FP8, class Out>
__device__ __forceinline__ void item_decode(uint32_t ncols, Lane &s, const uint4 *mp, Out &out) {
  const uint32_t nsteps = FP8 ? ncols : (ncols + 1) / 2;
  for (uint32_t gi = 0; gi * 16 < ncols; ++gi) {
    uint32_t mw[4] = {0u, 0u, 0u, 0u};
    if (!FP8) {
      const uint4 m = mp[gi * 64];
      mw[0] = m.x;
      mw[1] = m.y;
      mw[2] = m.z;
      mw[3] = m.w;
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

// Writes one row segment; elements of columns past ncols are dropped.
struct RowOut {
  uint8_t *dst;  // element (row, c0)
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
  uint32_t *region = s_code + wave * g.region_words;
  load_lut(g, s_lut);
  const bool active = item < g.n_items;
  if (active) stage_item(g, item, lane, region);
  __syncthreads();
  if (!active) return;
  const uint32_t rb = item / g.n_kspans, ks = item - rb * g.n_kspans;
  const uint32_t c0 = ks * g.cols, ncols = ks == g.n_kspans - 1 ? g.last_cols : g.cols;
  const int64_t row = (int64_t)rb * 64 + lane;
  Lane s{lds_addr(region) + 4 * lane, lds_addr(s_lut), 0u, g.r2s_lo, g.r2s_hi};
  const int64_t esz = FP8 ? 1 : 2;
  RowOut out{w + (row * ld + c0) * esz, ncols, row < g.n};
  item_decode<FP8>(ncols, s, FP8 ? nullptr : mant_base(g, rb, c0, lane), out);
}

// Thread t decodes row ids[t] (its lane's own stream column in LDS).
template <bool FP8>
__global__ __launch_bounds__(kThreads) void gather_kernel(Geom g, const int64_t *__restrict__ ids, int64_t n_ids,
                                                          uint8_t *__restrict__ out) {
  __shared__ uint32_t s_lut[NWC_LUT_ENTRIES];
  extern __shared__ uint32_t s_code[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t *region = s_code + wave * g.region_words;
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
    uint32_t *dst = region + lane;
    for (uint32_t r = 0; r < rows; ++r) dst[r * 64] = src[r * 64];
    const uint32_t c0 = ks * g.cols, ncols = ks == g.n_kspans - 1 ? g.last_cols : g.cols;
    Lane s{lds_addr(region) + 4 * lane, lds_addr(s_lut), 0u, g.r2s_lo, g.r2s_hi};
    RowOut o{out + (t * g.k + c0) * esz, ncols, live};
    if (valid) {
      item_decode<FP8>(ncols, s, FP8 ? nullptr : mant_base(g, rb, c0, L), o);
    } else if (live) {
      for (uint32_t c = 0; c < ncols * esz; ++c) o.dst[c] = 0;
    }
  }
}

Geom make_geom(const nwc_header_t &h, const void *d_blob) {
  Geom g;
  g.blob = (const uint8_t *)d_blob;
  g.n = h.n;
  g.k = h.k;
  g.cols = h.cols_per_item;
  g.n_rowblocks = h.n_rowblocks;
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

// Dynamic LDS: per wave, `chains` staged code regions (the table is static LDS).
size_t lds_bytes(const Geom &g, int chains) { return (size_t)kWaves * chains * g.region_words * 4; }

constexpr size_t kMaxDynamicLds = 48 * 1024;  // + 16 KiB static table = 64 KiB per workgroup

// Decode chains per wave for a BF16 matvec.  One: every wave of a typical
// matrix is resident at once, so a wave's lifetime sets the kernel time and a
// second chain only lengthens it.  NWC_CHAINS=2|4 selects more for experiments.
int matvec_chains(const Geom &g) {
  if (const char *e = getenv("NWC_CHAINS")) {
    const int v = atoi(e);
    if ((v == 1 || v == 2 || v == 4) && lds_bytes(g, v) <= kMaxDynamicLds) return v;
  }
  return 1;
}

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int launched() { return hipGetLastError() == hipSuccess ? NWC_OK : NWC_ERR_HIP; }

int read_header(const void *header, nwc_header_t &h) {
  if (!header) return NWC_ERR_ARG;
  memcpy(&h, header, sizeof h);
  return nwc_check_header(&h);
}

template <bool FP8, int NI, int D>
void launch_matvec(const Geom &g, hipStream_t s, const void *d_x, const float *d_scale, float *d_y, float *partial) {
  const uint32_t waves = (g.n_rowblocks + NI - 1) / NI * g.n_kspans;
  const dim3 grid((waves + kWaves - 1) / kWaves), block(kThreads);
  hipLaunchKernelGGL((matvec_kernel<FP8, NI, D>), grid, block, lds_bytes(g, NI), s, g,
                     (const uint32_t *)(g.blob + g.off_items), (const uint16_t *)d_x, d_scale, d_y, partial);
  if (g.n_kspans > 1)
    hipLaunchKernelGGL((reduce_kernel<FP8>), dim3((unsigned)((g.n * 16 + 255) / 256)), dim3(256), 0, s, partial,
                       g.n_kspans, g.n, d_scale, d_y);
}

// Mantissa prefetch ring depth (NWC_RING=1|2|4 overrides for experiments).
int ring_depth() {
  if (const char *e = getenv("NWC_RING")) {
    const int v = atoi(e);
    if (v == 1 || v == 2 || v == 4) return v;
  }
  return 2;
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
  if (need > 0) {
    if (!d_ws || !aligned(d_ws, 256)) return NWC_ERR_ARG;
    if (ws_bytes < need) return NWC_ERR_CAPACITY;
    partial = (float *)d_ws;
  }
  const Geom g = make_geom(h, d_blob);
  hipStream_t s = (hipStream_t)stream;
  if (fp8) {
    launch_matvec<true, 1, 1>(g, s, d_x, d_scale, d_y, partial);
  } else {
    const int ni = matvec_chains(g), d = ring_depth();
    if (ni == 1 && d == 1) launch_matvec<false, 1, 1>(g, s, d_x, d_scale, d_y, partial);
    else if (ni == 1 && d == 2) launch_matvec<false, 1, 2>(g, s, d_x, d_scale, d_y, partial);
    else if (ni == 1) launch_matvec<false, 1, 4>(g, s, d_x, d_scale, d_y, partial);
    else if (ni == 2) launch_matvec<false, 2, 2>(g, s, d_x, d_scale, d_y, partial);
    else launch_matvec<false, 4, 2>(g, s, d_x, d_scale, d_y, partial);
  }
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
    hipLaunchKernelGGL(dequant_kernel<true>, grid, block, lds_bytes(g, 1), s, g, (uint8_t *)d_w, ld);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, grid, block, lds_bytes(g, 1), s, g, (uint8_t *)d_w, ld);
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
    hipLaunchKernelGGL(gather_kernel<true>, grid, block, lds_bytes(g, 1), s, g, d_ids, n_ids, (uint8_t *)d_out);
  else
    hipLaunchKernelGGL(gather_kernel<false>, grid, block, lds_bytes(g, 1), s, g, d_ids, n_ids, (uint8_t *)d_out);
  return launched();
}

}  // extern "C"
