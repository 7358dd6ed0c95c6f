// gfx950 kernels of libnwc: fused decode + matvec, dequantization, gather.
//
// What is computed follows the "neural-weight-compression 0.9.0" PyPI page
// ("How it works": weights decoded in registers inside the matvec, fp32 row
// sums, dequantization and embedding lookup on the same decoder) and the
// "Qwen3-4B-NWC-fp8" model card (scale applied after the row sum).  The
// kernel design is this library's own, for CDNA4 wave64:
//
//  * One workgroup of W waves owns R whole rows: lane L of wave w decodes a
//    slice of C columns of row L/(64/R); the 64/R lanes of a row and the W
//    waves together cover the row (layout in nwc_format.h).  The row sum
//    finishes with a butterfly over the row's lanes and a sum over the waves
//    in LDS, in a fixed order: one kernel per matvec, no partial sums in
//    memory, no atomics.  (Rows longer than 16*64*C/R are split over several
//    workgroups whose partials a second small kernel sums.)
//  * A lane's decode chain is C/2 dependent steps (C <= 64), so a wave's
//    latency stays short and small matrices still get thousands of waves.
//  * Each wave's code streams are staged into LDS with direct 16-byte
//    HBM->LDS loads, lane L's stream in LDS column L (bank L mod 32: no
//    conflicts); the 16 KiB decode table is copied the same way, 1 KiB per
//    load, shared by the workgroup.
//  * Each step a lane reads 64 bits of its stream at its own bit position
//    (ds_read2st64), cuts a 12-bit peek with v_alignbit, and looks it up in the
//    decode table, which yields the two exponent/sign bytes of the next two
//    weights (BF16) or one whole value (fp8) plus the bits consumed.  v_perm
//    joins them with the raw mantissa bytes into a BF16 pair and
//    v_dot2c_f32_bf16 accumulates it in fp32.  Peeks the table cannot finish
//    (escapes, long pairs) take a wave-uniform branch to an exact decoder.
//  * Raw mantissa bytes and the lane's activations come straight from HBM
//    into registers (16-byte loads; a wave's mantissa load is one contiguous
//    KiB).  Activations past column K read as zero, and filler columns decode
//    to finite values, so padding adds exactly zero.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "nwc_check.h"

static_assert(offsetof(nwc_header_t, n) == 16 && offsetof(nwc_header_t, k) == 24 &&
                  offsetof(nwc_header_t, rows_per_wave) == 36 && offsetof(nwc_header_t, n_rowgroups) == 48 &&
                  offsetof(nwc_header_t, max_rows) == 56 && offsetof(nwc_header_t, escape_r) == 60 &&
                  offsetof(nwc_header_t, off_mant) == 88 &&
                  offsetof(nwc_header_t, off_code) == 96 && offsetof(nwc_header_t, rank_to_sym) == 128,
              "header word offsets read by the group kernel");

namespace {

constexpr int kWavesPerCu = 25;  // persistent grids: waves per compute unit
constexpr uint32_t kSelLo = 0x06010500u;   // {m[0], hiA, m[1], hiB}
constexpr uint32_t kSelHi = 0x06030502u;   // {m[2], hiA, m[3], hiB}
constexpr uint32_t kSelPair = 0x05040100u; // {a.b0, a.b1, b.b0, b.b1}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint32_t lds_u32;

struct Geom {
  const uint8_t *blob;
  int64_t n, k;
  uint32_t C, R, S, log2S, W, n_spans, n_rowgroups, n_items, region_words;
  uint32_t r2s_lo, r2s_hi;  // rank_to_sym[0..7], one byte each
  uint32_t huff;            // fp8 blob of the Huffman coder
  uint32_t code_words4;     // code plane bytes (a buffer range; the format keeps offsets below 2^32)
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
__device__ __forceinline__ uint32_t bf16_pair_exact(uint32_t col_base, uint32_t Q, uint32_t lo, uint32_t hi) {
  const uint64_t v = window64(col_base, Q + NWC_LEAD_BITS);
  uint32_t ha, la, hb, lb;
  bf16_code((uint32_t)v, lo, hi, ha, la);
  bf16_code((uint32_t)(v >> la), lo, hi, hb, lb);
  return (la + lb) | (ha << 8) | (hb << 16);
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

// Escape table of the fp8 decoder: an escape is 8 ones, then the byte's sign,
// 4-bit exponent field and 3-bit mantissa raw, so its 8 payload bits (stream
// bits 8..15 of the code) index a 256-entry table of decode-table entries
// {BF16 value, byte, 16 bits used}.  Each workgroup writes it into LDS right
// after the decode table (NWC_FP8_ESC_ENTRIES words); with it every fp8 code
// decodes from a table, escapes included.
constexpr uint32_t NWC_FP8_ESC_ENTRIES = 256;
__device__ __forceinline__ void build_fp8_escapes(uint32_t esc, uint32_t tid, uint32_t threads) {
  for (uint32_t p = tid; p < NWC_FP8_ESC_ENTRIES; p += threads) {
    const uint32_t b = ((p & 1u) << 7) | (((p >> 1) & 15u) << 3) | (p >> 5);
    *(lds_u32 *)(size_t)(esc + 4 * p) = fp8_to_bf16(b) | (b << 16) | (16u << 24);
  }
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
  for (int i = 0; i < NI; ++i) s[i].Q += e[i] & 0xFFu;
}

// Next fp8 code: returns {bf16 value, byte, bits}.  The escape table (after
// the decode table) answers for the peeks the decode table flags.
__device__ __forceinline__ uint32_t fp8_step(Lane &s) {
  const uint32_t a = word_addr(s.col, s.Q);
  const uint32_t W = __builtin_amdgcn_alignbit(lds_load(a + 256), lds_load(a), s.Q);
  const uint32_t e = lds_load(s.lut + (W & 0x3FFCu));
  const uint32_t x = lds_load(s.lut + NWC_LUT_BYTES + ((W >> 8) & 0x3FCu));  // payload = bits 10..17 of W
  const uint32_t v = (int)e < 0 ? x : e;
  s.Q += v >> 24;
  return v;
}

__device__ __forceinline__ uint32_t bf16_step(Lane &s) {
  Lane one[1] = {s};
  uint32_t e[1];
  bf16_steps<1>(one, e);
  s = one[0];
  return e[0];
}

// A lane's stream held in registers: a window of WN words (least significant
// first) whose next code starts at bit 2, as the stream's first code does.
// Each step shifts the window right by the bits it used, zeros coming in at
// the top, so the table peek is always bits 2..13 of word 0 and a step needs
// one LDS access (the table) instead of two.  A window of WN words holds the
// whole stream of an item with at most WN code rows.
template <int WN>
struct Win {
  uint32_t w[WN];
};

// Shift right by n mod 32 (the shifts use the low five bits of n; n is a
// decode-table entry or a code length, whose byte 0 is below 32).  Two words
// shift as one 64-bit value: one instruction instead of two.
template <int WN>
__device__ __forceinline__ void win_shift(Win<WN> &s, uint32_t n) {
  if constexpr (WN == 2) {
    const uint64_t v = ((((uint64_t)s.w[1]) << 32) | s.w[0]) >> (n & 63u);
    s.w[0] = (uint32_t)v;
    s.w[1] = (uint32_t)(v >> 32);
  } else {
#pragma unroll
    for (int i = 0; i + 1 < WN; ++i) s.w[i] = __builtin_amdgcn_alignbit(s.w[i + 1], s.w[i], n);
    s.w[WN - 1] = s.w[WN - 1] >> (n & 31u);
  }
}

// Next two BF16 codes from the window: a {bits, hiA, hiB} entry.  When a lane
// of the wave meets an escape or a pair longer than the peek, every lane takes
// the exact decode; it shifts out code A itself (a pair may use 32 bits) and
// leaves the bits of code B in the entry for the common shift.
template <int WN>
__device__ __forceinline__ uint32_t bf16_step_win(Win<WN> &s, uint32_t lut, uint32_t lo, uint32_t hi) {
  uint32_t e = lds_load(lut + (s.w[0] & 0x3FFCu));
  if (__builtin_expect(__any((int)e < 0), 0)) {
    const uint64_t v = ((((uint64_t)s.w[1]) << 32) | s.w[0]) >> NWC_LEAD_BITS;
    uint32_t ha, la, hb, lb;
    bf16_code((uint32_t)v, lo, hi, ha, la);
    bf16_code((uint32_t)(v >> la), lo, hi, hb, lb);
    win_shift(s, la);
    e = lb | (ha << 8) | (hb << 16);
  }
  win_shift(s, e);
  return e;
}

// Next fp8 code from the window: {bf16 value, byte, bits}.  The escape table
// answers for the peeks the decode table flags (codes longer than the peek,
// about 1 % of them); the wave reads it only when one of its lanes needs it.
// Measured on MI355X (9728 x 2560): the bank conflicts of the table reads
// bound the fp8 decode, and skipping the unneeded ones is 11 % faster.
template <int WN>
__device__ __forceinline__ uint32_t fp8_step_win(Win<WN> &s, uint32_t lut) {
  const uint32_t e = lds_load(lut + (s.w[0] & 0x3FFCu));
  uint32_t v = e;
  if (__any((int)e < 0)) {
    const uint32_t x = lds_load(lut + NWC_LUT_BYTES + ((s.w[0] >> 8) & 0x3FCu));  // payload = bits 10..17
    v = (int)e < 0 ? x : e;
  }
  win_shift(s, v >> 24);
  return v;
}

// ----------------------------------------------------------------- staging
typedef __attribute__((address_space(3))) void lds_void;

// 1 KiB global -> LDS (byte address dst) straight into LDS (no registers),
// lane L moving bytes [16L, 16L+16); lanes past `bytes` do nothing.
__device__ __forceinline__ void dma_1k(const uint8_t *src, uint32_t dst, uint32_t bytes, uint32_t lane) {
  if (lane * 16 < bytes)
    __builtin_amdgcn_global_load_lds(src + lane * 16, (lds_void *)(size_t)dst, 16, 0, 0);
}

// This wave's share of a copy global -> LDS, 1 KiB per instruction.
__device__ __forceinline__ void dma_to_lds(const uint8_t *src, uint32_t dst, uint32_t bytes, uint32_t lane) {
  for (uint32_t off = 0; off < bytes; off += 1024) dma_1k(src + off, dst + off, bytes - off, lane);
}

// The decode table in 16 pieces of 1 KiB; wave w of `waves` copies pieces w, w+waves, ...
__device__ __forceinline__ void dma_lut(const Geom &g, uint32_t lut, uint32_t wave, uint32_t waves, uint32_t lane) {
  for (uint32_t p = wave; p < NWC_LUT_BYTES / 1024; p += waves)
    dma_1k(g.blob + g.off_lut + p * 1024, lut + p * 1024, 1024, lane);
}

__device__ __forceinline__ void lds_store(uint32_t byte_addr, uint32_t v) { *(lds_u32 *)(size_t)byte_addr = v; }

// Waits as builtins, which the compiler's own wait placement takes into
// account (it does not read inline assembly): vmcnt(0), lgkmcnt(0).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Buffer resource word 3 for untyped 32-bit accesses (data format 32).
constexpr int kBufWord3 = 0x00020000;

// The blob's bytes are read once per call, so the streaming kernels (matvec,
// dequant, matrix-core batch) mark its loads non-temporal (the nt cache-policy
// bit; kLoadNT for buffer loads, ld_nt for 16-byte loads).  Measured on
// MI355X: a streaming read of 1 GiB moves 7.15 TB/s with non-temporal loads
// against 6.54 TB/s without (75 MiB: 6.19 vs 5.75 TB/s), and the Qwen3-4B
// layer set went from 1.40 to 1.33 ms.  The decode table and the activations,
// which every workgroup reads, keep the default policy, and so does the
// gather (4096 ids: 11.1 us with non-temporal loads, 10.8 us without).
constexpr int kLoadNT = 2;
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4 *p) {
  const u32x4_nt v = __builtin_nontemporal_load((const u32x4_nt *)p);
  return uint4{v.x, v.y, v.z, v.w};
}

// The first PR code rows of an item, this lane's column, fetched into
// registers while the wave still decodes its previous item.  The loads go
// through a buffer resource sized to the item (rows * 256 bytes): rows past the
// item's end read as zero without a memory access and become its guard rows.
// rows == 0 fetches nothing (no next item).
template <int PR>
__device__ __forceinline__ void fetch_code_ahead(const uint8_t *code, uint32_t off, uint32_t rows, uint32_t lane,
                                                 uint32_t (&w)[PR]) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(code + off), (short)0, (int)(rows * 256), kBufWord3);
  // Keeps the row offsets in the instructions' offset fields instead of one
  // register per row (the compiler would hoist the sums out of the loop).
  uint32_t col = 4 * lane;
  asm volatile("" : "+v"(col));
#pragma unroll
  for (int j = 0; j < PR; ++j) w[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, col + j * 256, 0, kLoadNT);
}

// Puts a fetched item into the wave's LDS region: the PR register rows (the
// rows the region holds), then, for an item longer than PR - 2 rows, its other
// rows straight from memory and the two zero guard rows.  col is the item lane
// whose stream this lane fetched (its column of the region; the lane itself
// except in the matrix-core kernel); lane moves its share of the copy.
template <int PR>
__device__ __forceinline__ void commit_code_ahead(const uint8_t *code, uint32_t off, uint32_t rows,
                                                  uint32_t region_rows, uint32_t region, uint32_t lane,
                                                  const uint32_t (&w)[PR], uint32_t col) {
#pragma unroll
  for (int j = 0; j < PR; ++j)
    if ((uint32_t)j < region_rows) lds_store(region + j * 256 + 4 * col, w[j]);
  if (rows + NWC_GUARD_ROWS > (uint32_t)PR) {
    if (rows > (uint32_t)PR) dma_to_lds(code + off + PR * 256, region + PR * 256, (rows - PR) * 256, lane);
    lds_store(region + rows * 256 + 4 * col, 0u);
    lds_store(region + (rows + 1) * 256 + 4 * col, 0u);
    wait_vm0();
  }
}

// Activation pairs of 16 columns from column c; columns at or past k are 0.
struct X16 {
  uint32_t v[8];
};
__device__ __forceinline__ X16 load_x16(const uint16_t *x, int64_t c, int64_t k) {
  X16 r;
  if (c + 16 <= k) {
    const uint4 *p = (const uint4 *)(x + c);
    const uint4 a = p[0], b = p[1];
    r = X16{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = c + 2 * j < k ? x[c + 2 * j] : 0u;
      const uint32_t hi = c + 2 * j + 1 < k ? x[c + 2 * j + 1] : 0u;
      r.v[j] = lo | (hi << 16);
    }
  }
  return r;
}

__device__ __forceinline__ uint32_t dword_of(const uint4 &m, int i) {
  return i == 0 ? m.x : i == 1 ? m.y : i == 2 ? m.z : m.w;
}

// Mantissa chunk 0 of lane L of an item; chunk j is 64 uint4 further.
__device__ __forceinline__ const uint4 *mant_base(const Geom &g, uint32_t item, uint32_t L) {
  return (const uint4 *)(g.blob + g.off_mant + (uint64_t)item * 64 * g.C) + L;
}

// Where lane `lane` of wave `wave` in workgroup `grp` sits in the matrix.
struct Place {
  uint32_t item, span, row_group, r, s;
  int64_t row, c0;
};
__device__ __forceinline__ Place place(const Geom &g, uint32_t grp, uint32_t wave, uint32_t lane) {
  Place p;
  p.item = grp * g.W + wave;
  p.row_group = grp / g.n_spans;
  p.span = grp - p.row_group * g.n_spans;
  p.s = lane & (g.S - 1u);
  p.r = lane >> g.log2S;
  p.row = (int64_t)p.row_group * g.R + p.r;
  p.c0 = (int64_t)((p.span * g.W + wave) * g.S + p.s) * g.C;
  return p;
}

// ----------------------------------------------------------------- matvec
// Row sums of this lane's slice against B activation rows: NG groups of 16
// columns, 8 two-code steps each; every decoded pair of weights is used B
// times.  Each row's sum is formed in the same order whatever B is.
template <int NG, int B, class Step>
__device__ __forceinline__ void slice_dot_bf16_rows(Step step, const uint4 (&m)[NG], const X16 (&xv)[B][NG],
                                                    float (&v)[B]) {
  float a0[B], a1[B];
#pragma unroll
  for (int b = 0; b < B; ++b) a0[b] = a1[b] = 0.f;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t e = step();
      const uint32_t p = __builtin_amdgcn_perm(e, dword_of(m[gi], j >> 1), (j & 1) ? kSelHi : kSelLo);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (j & 1)
          a1[b] = dot2(p, xv[b][gi].v[j], a1[b]);
        else
          a0[b] = dot2(p, xv[b][gi].v[j], a0[b]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) v[b] = a0[b] + a1[b];
}

// The lane's stream in the wave's LDS region.
template <int NG, int B>
__device__ __forceinline__ void slice_dot_bf16(Lane &st, const uint4 (&m)[NG], const X16 (&xv)[B][NG], float (&v)[B]) {
  slice_dot_bf16_rows<NG, B>([&] { return bf16_step(st); }, m, xv, v);
}

// The lane's stream in a register window.
template <int NG, int B, int WN>
__device__ __forceinline__ void slice_dot_bf16_win(Win<WN> &s, uint32_t lut, uint32_t lo, uint32_t hi,
                                                   const uint4 (&m)[NG], const X16 (&xv)[B][NG], float (&v)[B]) {
  slice_dot_bf16_rows<NG, B>([&] { return bf16_step_win(s, lut, lo, hi); }, m, xv, v);
}

template <int NG, class Step>
__device__ __forceinline__ float slice_dot_fp8_codes(Step step, const X16 (&xv)[NG]) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t ea = step();
      const uint32_t eb = step();
      const uint32_t p = __builtin_amdgcn_perm(eb, ea, kSelPair);
      if (j & 1)
        a1 = dot2(p, xv[gi].v[j], a1);
      else
        a0 = dot2(p, xv[gi].v[j], a0);
    }
  }
  return a0 + a1;
}

// Two fp8 codes of a Huffman-coded stream per window shift: no code escapes
// the 12-bit peek, so the second code's peek is the first two words shifted by
// the first code's length (one v_alignbit), and the window shifts once by both
// lengths (at most 24 bits).  Per pair of weights: 2 table reads and 8 + WN
// other instructions, against 2 x (4 + WN) for two single steps with their
// escape tests.  Returns the two values as a BF16 pair.
template <int WN>
__device__ __forceinline__ uint32_t fp8_pair_win(Win<WN> &s, uint32_t lut) {
  const uint32_t ea = lds_load(lut + (s.w[0] & 0x3FFCu));
  const uint32_t la = ea >> 24;
  const uint32_t eb = lds_load(lut + (__builtin_amdgcn_alignbit(s.w[1], s.w[0], la) & 0x3FFCu));
  win_shift(s, la + (eb >> 24));
  return __builtin_amdgcn_perm(eb, ea, kSelPair);
}

template <int NG, int WN>
__device__ __forceinline__ float slice_dot_fp8_pairs_win(Win<WN> &s, uint32_t lut, const X16 (&xv)[NG]) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t p = fp8_pair_win(s, lut);
      if (j & 1)
        a1 = dot2(p, xv[gi].v[j], a1);
      else
        a0 = dot2(p, xv[gi].v[j], a0);
    }
  }
  return a0 + a1;
}

// The lane's stream in the wave's LDS region.
template <int NG>
__device__ __forceinline__ float slice_dot_fp8(Lane &st, const X16 (&xv)[NG]) {
  return slice_dot_fp8_codes<NG>([&] { return fp8_step(st); }, xv);
}

// The lane's stream in a register window.
template <int NG, int WN>
__device__ __forceinline__ float slice_dot_fp8_win(Win<WN> &s, uint32_t lut, const X16 (&xv)[NG]) {
  return slice_dot_fp8_codes<NG>([&] { return fp8_step_win(s, lut); }, xv);
}

// Partial sums live at [row][column span], each row padded to a multiple of
// 4 spans (16-byte loads in the reduction).
__device__ __forceinline__ uint32_t spans_pad(uint32_t n_spans) { return (n_spans + 3u) & ~3u; }

// Sum of the S adjacent lanes of each row (S a power of two, 1..64), left in
// the row's last lane (lane r*S + S-1); other lanes hold partial windows.
// DPP adds in a fixed order: row_shr 1, 2, 4, 8 sum windows of up to 16
// lanes inside each 16-lane row, row_bcast:15 / row_bcast:31 join rows.
__device__ __forceinline__ float row_sum_lanes(float a, uint32_t S) {
  if (S >= 2) a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0x111, 0xF, 0xF, true));
  if (S >= 4) a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0x112, 0xF, 0xF, true));
  if (S >= 8) a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0x114, 0xF, 0xF, true));
  if (S >= 16) a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0x118, 0xF, 0xF, true));
  if (S >= 32) a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0x142, 0xA, 0xF, false));
  if (S >= 64) a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0x143, 0xC, 0xF, false));
  return a;
}

// Geometry of the matrix-vector product resolved on the host, the part a
// wave does not need at once (the kernel takes the rest as leading scalar
// arguments): the mantissa plane and 32-bit sizes (the format caps n and k at
// 2^31).  All of it is wave-uniform and lives in scalar registers, which also
// bound how many waves a SIMD takes.
struct MvArgs {
  const uint8_t *mant;  // mantissa plane
  uint32_t n, R, n_spans, region_words, r2s_lo, r2s_hi, groups_cap;
  uint32_t ldx, ldy;  // elements between the activation rows / output rows of a batch
  uint32_t huff;      // fp8 blob of the Huffman coder: no escapes
};

// y[row] (times the fp8 row scale) with one span per row, else the span's
// partial sum at [row][spans_pad(n_spans)].
template <bool FP8, bool SPLIT>
__device__ __forceinline__ void store_out(const MvArgs &a, uint32_t row, uint32_t span, float v,
                                          const float *__restrict__ scale, float *__restrict__ y,
                                          float *__restrict__ partial, uint32_t b = 0) {
  if (row >= a.n) return;
  if (!SPLIT)
    y[(uint64_t)b * a.ldy + row] = FP8 ? v * scale[row] : v;
  else
    partial[(uint64_t)row * spans_pad(a.n_spans) + span] = v;
}

template <int NG, int B>
__device__ __forceinline__ void load_x_slice(const uint16_t *__restrict__ x, uint32_t ldx, uint32_t k,
                                             X16 (&xv)[B][NG], uint32_t c0) {
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int j = 0; j < NG; ++j) xv[b][j] = load_x16(x + (uint64_t)b * ldx, (int64_t)c0 + 16 * j, k);
}

// Persistent workgroups: workgroup b decodes the groups (row group, column
// span) b, b + grid, b + 2*grid, ... of the G = n_rowgroups * n_spans.  The
// decode table (and, with one span per row, the activations) is staged once
// per workgroup.  Each wave fetches the code rows of its next item into
// registers while it decodes the current one, so after the first item the
// memory system streams while the waves decode.  Row sums go to per-group LDS
// slots; the outputs are written once every wave is done, each row adding its
// W wave partials in wave order.
//
// What a wave needs first (item table, code plane, decode table, activations,
// the group count and stride, the item shape) comes as the leading scalar
// arguments: the build asks for kernel-argument preloading, so gfx950 puts
// them in scalar registers at wave launch.  Measured on MI355X, a launch's
// waves otherwise wait up to ~2.5 us for their arguments through the scalar
// cache.  The buffers are __restrict__, so the compiler may read the item
// table through the scalar cache.
// The decode table into LDS, 1 KiB per direct load; wave w of W copies
// pieces w, w + W, ...  Issued first by every matvec workgroup: nothing it
// needs has to arrive before.
__device__ __forceinline__ void stage_lut(const uint8_t *lut, uint32_t *s_lut, uint32_t W, uint32_t wave,
                                          uint32_t lane) {
  for (uint32_t p = wave; p < NWC_LUT_BYTES / 1024; p += W)
    dma_1k(lut + p * 1024, lds_addr(s_lut) + p * 1024, 1024, lane);
}

// The body of a matvec workgroup: `first` is its index among the `grid`
// workgroups that share this matrix; off0/rows0 are this wave's first
// item-table entry, which the caller reads before calling (scalar loads issued
// before the decode table's copy; the body waits for them right after it).
// The table copy is issued here, where `lut`, `items` and `code` are
// restrict-qualified: the compiler then knows that the copy does not write the
// item table and keeps the item-table reads in the loop scalar loads.  s_lut: the static decode table (and
// fp8 escape table); s_dyn: one code region per wave, then groups_cap slots of
// W*R row sums (matvec_lds on the host sizes it).
// Issue priority by work left.  The workgroups sharing a compute unit start
// one after another, and by default the older waves win the issue slots, so
// the first workgroups finish early and the last ones run alone at the end
// of the launch.  Before each of its items a wave of a multi-item workgroup
// raises its priority with the items it has left (5 or more: 3, 3-4: 2,
// 2: 1, the last: 0), so the workgroups on a CU finish closer together.
// Measured on MI355X (Qwen3-4B layer set): 3647-3671 -> 3713-3735 GB/s; the
// one-item workgroups keep the default priority (setting it cost 0.1 us on
// the 1024-row matrices).  The dequantization, bound by its stores, was
// slower with it (300 -> 302-306 us on the 151936 x 2560 table) and keeps
// the default.
__device__ __forceinline__ void issue_priority(uint32_t n_items, uint32_t i) {
  if (n_items <= 1) return;
  const uint32_t rem = n_items - i;
  if (rem >= 5)
    __builtin_amdgcn_s_setprio(3);
  else if (rem >= 3)
    __builtin_amdgcn_s_setprio(2);
  else if (rem == 2)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

template <bool FP8, int NG, bool SPLIT, int B, int LS = -1>
__device__ __forceinline__ void matvec_body(const uint32_t *__restrict__ items, const uint8_t *__restrict__ code,
                                            const uint8_t *__restrict__ lut, const uint16_t *__restrict__ x,
                                            uint32_t n_groups, uint32_t W, uint32_t grid, uint32_t first, uint32_t k,
                                            uint32_t log2S_arg, const MvArgs &a, const float *__restrict__ scale,
                                            float *__restrict__ y, float *__restrict__ partial, uint32_t *s_lut,
                                            uint32_t *s_dyn, uint32_t off0, uint32_t rows0) {
  constexpr uint32_t C = 16 * NG;
  // Lanes per row as a constant where the caller knows it (the row sums then
  // take no branches).
  const uint32_t log2S = LS >= 0 ? (uint32_t)LS : log2S_arg;
  // Code rows fetched ahead: a BF16 item's rows and its guard rows, typically;
  // an fp8 item (6.75 bits per weight) takes 4 to 6 rows of 16-column slices.
  constexpr int PR = FP8 ? 2 * NG + 4 : 2 * NG + 2;
  constexpr uint32_t kWinMax = FP8 ? 6u : 4u;  // longest item decoded from registers
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The table copy first: it needs nothing from memory, while the group
  // count below may come from the blob's header (a scalar load the copy would
  // otherwise wait for).
  stage_lut(lut, s_lut, W, wave, lane);
  // Workgroup b takes groups b, b + grid, b + 2*grid, ...: at any time the
  // workgroups read neighbouring items, so the machine streams the planes in
  // order.
  // A scalar: the division would otherwise leave it, and every test of the
  // item count, in vector registers.
  const uint32_t n_mine = __builtin_amdgcn_readfirstlane((n_groups - first + grid - 1) / grid);
  const uint32_t region = lds_addr(s_dyn) + wave * a.region_words * 4;  // LDS byte address
  const uint32_t region_rows = a.region_words >> 6;
  float *red = (float *)(s_dyn + W * a.region_words);  // [group][wave][activation row][R]
  const uint32_t S = 1u << log2S;
  const uint32_t r = lane >> log2S, lane_c = (lane & (S - 1u)) * C;  // row in group, column in slice run
  const bool row_lane = (lane & (S - 1u)) == S - 1u;

  // Waits for the first item-table entry and the shape words (which the
  // grouped kernel reads from the blob's header) here, once, right after the
  // table copy is issued, instead of where the compiler would put the first
  // use (after the start barrier, one memory round trip later).
  asm volatile("" ::"s"(off0), "s"(rows0), "s"(a.r2s_lo), "s"(a.r2s_hi), "s"(a.R), "s"(a.region_words), "s"(a.n));
  if (FP8 && !a.huff) build_fp8_escapes(lds_addr(s_lut) + NWC_LUT_BYTES, threadIdx.x, blockDim.x);
  // (row group, span) of the current group, stepped without a division.
  uint32_t rg = SPLIT ? first / a.n_spans : first, sp = first - rg * a.n_spans;
  const uint32_t step_rg = SPLIT ? grid / a.n_spans : grid, step_sp = grid - step_rg * a.n_spans;
  uint32_t ahead[PR];
  fetch_code_ahead<PR>(code, off0, rows0, lane, ahead);
  wait_vm0();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  // The activations after the barrier: the first decode does not need them,
  // and every workgroup of a launch reads the same few KiB at its start.
  // Measured on MI355X, waiting for them with the decode table made the
  // Qwen3-4B layer set 3.5 % slower (1.484 vs 1.433 ms per sweep).
  X16 xv[B][NG];
  load_x_slice<NG, B>(x, a.ldx, k, xv, ((sp * W + wave) << log2S) * C + lane_c);

  // The item-table entry of the item whose rows are in flight, read when they
  // were fetched.
  uint32_t off_next = off0, rows_next = rows0;
  for (uint32_t i = 0, grp = first; i < n_mine; ++i, grp += grid) {
    const uint32_t item = grp * W + wave;
    issue_priority(n_mine, i);
    // Items of at most kWinMax code rows (BF16: 4, fp8: 6) decode from a
    // register window of that many words (at least two); longer ones from the
    // wave's LDS region.
    const uint32_t rows = rows_next, off = off_next;
    const uint32_t wn = rows > kWinMax ? 0u : rows < 2u ? 2u : rows;
    if (SPLIT && grp != first) load_x_slice<NG, B>(x, a.ldx, k, xv, ((sp * W + wave) << log2S) * C + lane_c);
    uint32_t cur[kWinMax];
#pragma unroll
    for (uint32_t j = 0; j < kWinMax; ++j) cur[j] = ahead[j];
    if (wn == 0) commit_code_ahead<PR>(code, off, rows, region_rows, region, lane, ahead, lane);
    // Mantissas of this item, then the next item's code rows: the decode below
    // needs neither, so both stream in while it runs (the compiler waits for
    // the mantissas at the multiply-adds, which it places after the decode
    // steps, and for the code rows where the next item starts).
    uint4 m[NG];
    if (!FP8) {
      const uint4 *mp = (const uint4 *)(a.mant + (uint64_t)item * (64 * C)) + lane;
#pragma unroll
      for (int j = 0; j < NG; ++j) m[j] = ld_nt(mp + j * 64);
    }
    {
      const bool more = i + 1 < n_mine;
      const uint32_t nx = more ? item + grid * W : item;
      off_next = items[2 * nx];
      rows_next = more ? items[2 * nx + 1] : 0u;
      fetch_code_ahead<PR>(code, off_next, rows_next, lane, ahead);
    }
    float v[B];
    auto run_win = [&](auto &win) {
      if constexpr (FP8)
        v[0] = a.huff ? slice_dot_fp8_pairs_win<NG>(win, lds_addr(s_lut), xv[0])
                      : slice_dot_fp8_win<NG>(win, lds_addr(s_lut), xv[0]);
      else
        slice_dot_bf16_win<NG, B>(win, lds_addr(s_lut), a.r2s_lo, a.r2s_hi, m, xv, v);
    };
    if (wn == 2) {
      Win<2> win{{cur[0], cur[1]}};
      run_win(win);
    } else if (wn == 3) {
      Win<3> win{{cur[0], cur[1], cur[2]}};
      run_win(win);
    } else if (wn == 4) {
      Win<4> win{{cur[0], cur[1], cur[2], cur[3]}};
      run_win(win);
    } else if (FP8 && wn == 5) {
      Win<5> win{{cur[0], cur[1], cur[2], cur[3], cur[kWinMax > 4 ? 4 : 0]}};
      run_win(win);
    } else if (FP8 && wn == 6) {
      Win<6> win{{cur[0], cur[1], cur[2], cur[3], cur[kWinMax > 4 ? 4 : 0], cur[kWinMax > 5 ? 5 : 0]}};
      run_win(win);
    } else {
      Lane st{region + 4 * lane, lds_addr(s_lut), 0u, a.r2s_lo, a.r2s_hi};
      if (FP8)
        v[0] = slice_dot_fp8<NG>(st, xv[0]);
      else
        slice_dot_bf16<NG, B>(st, m, xv, v);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      v[b] = row_sum_lanes(v[b], S);
      if (row_lane) red[((i * W + wave) * B + b) * a.R + r] = v[b];
    }
    if (!SPLIT) {
      rg += grid;
    } else {
      sp += step_sp;
      rg += step_rg;
      if (sp >= a.n_spans) {
        sp -= a.n_spans;
        ++rg;
      }
    }
  }

  // Outputs: row (group i, activation row b, r) = sum over waves w of
  // slot[i][w][b][r], w ascending.
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  const uint32_t log2R = 6 - log2S;
  const uint32_t n_out = (n_mine * B) << log2R;
  for (uint32_t t = threadIdx.x; t < n_out; t += blockDim.x) {
    const uint32_t ib = t >> log2R, rr = t & (a.R - 1u);
    const uint32_t i = ib / B, b = ib - i * B;
    const float *slot = red + (i * W * B + b) * a.R + rr;
    float sum = 0.f;
    for (uint32_t w = 0; w < W; ++w) sum += slot[w * B * a.R];
    const uint32_t grp = first + i * grid, grow = SPLIT ? grp / a.n_spans : grp;
    store_out<FP8, SPLIT>(a, grow * a.R + rr, grp - grow * a.n_spans, sum, scale, y, partial, b);
  }
}

template <bool FP8, int NG, bool SPLIT, int B, int LS = -1>
__global__ __launch_bounds__(1024) void matvec_kernel(const uint32_t *__restrict__ items, const uint8_t *__restrict__ code,
                                                      const uint8_t *__restrict__ lut, const uint16_t *__restrict__ x,
                                                      uint32_t n_groups, uint32_t W, uint32_t grid, uint32_t k,
                                                      uint32_t log2S, const MvArgs a,
                                                      const float *__restrict__ scale, float *__restrict__ y,
                                                      float *__restrict__ partial) {
  __shared__ uint32_t s_lut[NWC_LUT_ENTRIES + (FP8 ? NWC_FP8_ESC_ENTRIES : 0)];
  extern __shared__ uint32_t s_dyn[];
  const uint32_t it = blockIdx.x * W + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t off0 = items[2 * it], rows0 = items[2 * it + 1];
  matvec_body<FP8, NG, SPLIT, B, LS>(items, code, lut, x, n_groups, W, grid, blockIdx.x, k, log2S, a, scale, y,
                                     partial, s_lut, s_dyn, off0, rows0);
}

// Several matrices of one work-item shape (elem, C, R, W; rows within one
// workgroup) in one launch, each with its own activation and output: the
// workgroups [begin[m], begin[m + 1]) run matrix m as the single-matrix kernel
// runs it on a grid of that many workgroups, so each output is bit-equal to
// the one nwc_matvec gives.
//
// What the first loads need comes in the leading scalar arguments, which
// gfx950 preloads into scalar registers at wave launch: the count, W and
// log2 S, the first workgroups of matrices 1 and 2, and the blob and
// activation of matrices 0..2.  Everything else about a matrix is read from
// its blob's header (one scalar load, issued beside the first item-table
// read, so the first code rows wait no longer than in the single-matrix
// kernel) or, for the output and the fp8 scales needed only at the end, from
// the argument segment.  Matrices 3 and up take their blob and activation
// from the argument segment too.
constexpr int kGroupMax = NWC_GROUP_MAX;
static_assert(NWC_GROUP_MAX < 16 && NWC_MAX_WAVES < 32, "group head packs the count in 4 bits and W in 5");
constexpr uint32_t kGroupPreloaded = 3;
struct GroupTail {
  uint32_t begin[kGroupMax + 1];  // first workgroup of each matrix; begin[count] = grid
  const uint8_t *blob[kGroupMax];
  const uint16_t *x[kGroupMax];
  const float *scale[kGroupMax];
  float *y[kGroupMax];
};

template <bool FP8, int NG, int LS = -1>
__global__ __launch_bounds__(1024) void matvec_group_kernel(uint32_t head, uint32_t begins,
                                                            const uint8_t *__restrict__ blob0,
                                                            const uint8_t *__restrict__ blob1,
                                                            const uint8_t *__restrict__ blob2,
                                                            const uint16_t *__restrict__ x0,
                                                            const uint16_t *__restrict__ x1,
                                                            const uint16_t *__restrict__ x2, const GroupTail tail) {
  __shared__ uint32_t s_lut[NWC_LUT_ENTRIES + (FP8 ? NWC_FP8_ESC_ENTRIES : 0)];
  extern __shared__ uint32_t s_dyn[];
  // head: count | W << 4 | log2 S << 9 | from_tail << 12 | grid << 13;
  // begins: first workgroup of matrix 1 | of matrix 2 << 16.  from_tail: the
  // first workgroups do not fit those fields and come from the tail.
  const uint32_t count = head & 15u, W = (head >> 4) & 31u, log2S = (head >> 9) & 7u;
  const uint32_t wg = blockIdx.x, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t m, beg, end;
  const uint8_t *blob;
  const uint16_t *x;
  if (count <= kGroupPreloaded && !((head >> 12) & 1u)) {
    const uint32_t all = head >> 13;
    const uint32_t b1 = count > 1 ? begins & 0xFFFFu : all, b2 = count > 2 ? begins >> 16 : all;
    m = wg >= b2 ? 2u : wg >= b1 ? 1u : 0u;
    beg = m == 0 ? 0u : m == 1 ? b1 : b2;
    end = m == 0 ? b1 : m == 1 ? b2 : all;
    blob = m == 0 ? blob0 : m == 1 ? blob1 : blob2;
    x = m == 0 ? x0 : m == 1 ? x1 : x2;
  } else {
    m = 0;
    for (uint32_t i = 1; i < count; ++i)
      if (wg >= tail.begin[i]) m = i;
    beg = tail.begin[m];
    end = tail.begin[m + 1];
    blob = tail.blob[m];
    x = tail.x[m];
  }
  // The first item-table entry and the header fields, read before anything
  // else (scalar loads: before the decode table's copy, which the compiler
  // would count as a write that could alias them); the body issues the copy
  // and then waits for all of them at once.  The item table and the decode
  // table sit at fixed offsets in the blob.
  const uint32_t *items = (const uint32_t *)(blob + NWC_HEADER_BYTES + NWC_LUT_BYTES);
  const uint32_t it = (wg - beg) * W + wave;
  const uint32_t off0 = items[2 * it], rows0 = items[2 * it + 1];
  // Header fields as 32-bit words (nwc_header_t: n at word 4, k at 6, R at 9,
  // row groups at 12, max_rows at 14, escape_r at 15, off_mant at 22-23,
  // off_code at 24-25, rank_to_sym at 32); n and k are below 2^31.
  const uint32_t *hw = (const uint32_t *)blob;
  const uint32_t n = hw[4], k = hw[6], R = hw[9], n_groups = hw[12], max_rows = hw[14];
  const uint32_t huff = FP8 ? hw[15] == 0 : 0u;
  const uint32_t om_lo = hw[22], om_hi = hw[23], oc_lo = hw[24], oc_hi = hw[25];
  const uint32_t r2s_lo = hw[32], r2s_hi = hw[33];
  const uint64_t off_mant = ((uint64_t)om_hi << 32) | om_lo, off_code = ((uint64_t)oc_hi << 32) | oc_lo;
  const uint32_t grid = end - beg;
  MvArgs a;
  a.mant = blob + off_mant;
  a.n = n;
  a.R = R;
  a.n_spans = 1;
  a.region_words = (max_rows + NWC_GUARD_ROWS) * 64;
  a.r2s_lo = r2s_lo;
  a.r2s_hi = r2s_hi;
  a.groups_cap = (n_groups + grid - 1) / grid;
  a.ldx = 0;
  a.ldy = 0;
  a.huff = huff;
  matvec_body<FP8, NG, false, 1, LS>(items, blob + off_code, blob + NWC_HEADER_BYTES, x, n_groups, W, grid, wg - beg,
                                     k, log2S, a, tail.scale[m], tail.y[m], nullptr, s_lut, s_dyn, off0, rows0);
}

// y[row] = (scale[row] *) sum over column spans of the partials, 16 threads
// per row: thread j sums 16-byte chunks j, j+16, ... in order, then a fixed
// butterfly over the 16 threads.  Same order every call.
template <bool FP8>
__global__ __launch_bounds__(256) void reduce_kernel(const float *__restrict__ partial, uint32_t n_spans, int64_t n,
                                                     const float *__restrict__ scale, float *__restrict__ y) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t >> 4;
  const uint32_t j = (uint32_t)t & 15u;
  const uint32_t kp = spans_pad(n_spans);
  float sum = 0.f;
  if (row < n) {
    const float4 *p = (const float4 *)(partial + (uint64_t)row * kp);
    for (uint32_t c = j; c < kp / 4; c += 16) {
      const float4 v = p[c];
      sum += v.x;
      if (4 * c + 1 < n_spans) sum += v.y;
      if (4 * c + 2 < n_spans) sum += v.z;
      if (4 * c + 3 < n_spans) sum += v.w;
    }
  }
  sum += __shfl_xor(sum, 8, 16);
  sum += __shfl_xor(sum, 4, 16);
  sum += __shfl_xor(sum, 2, 16);
  sum += __shfl_xor(sum, 1, 16);
  if (j == 0 && row < n) y[row] = FP8 ? sum * scale[row] : sum;
}

// ----------------------------------------------------------------- dequant / gather
// Writes the 16 decoded elements of one column group of a row (BF16 pairs
// or fp8 bytes) to dst = &out[row][c]; only columns below `left` are real.
template <bool FP8>
__device__ __forceinline__ void put_group(uint8_t *dst, const uint32_t (&v)[8], int64_t left, bool vec) {
  if (left <= 0) return;
  if (FP8) {
    if (left >= 16 && vec) {
      *(uint4 *)dst = make_uint4(v[0], v[1], v[2], v[3]);
    } else {
      for (int i = 0; i < 16 && i < left; ++i) dst[i] = (uint8_t)(v[i >> 2] >> (8 * (i & 3)));
    }
  } else {
    if (left >= 16 && vec) {
      ((uint4 *)dst)[0] = make_uint4(v[0], v[1], v[2], v[3]);
      ((uint4 *)dst)[1] = make_uint4(v[4], v[5], v[6], v[7]);
    } else {
      uint16_t *d = (uint16_t *)dst;
      for (int i = 0; i < 16 && i < left; ++i) d[i] = (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
    }
  }
}

// Decodes NG groups of a lane's slice; hands each group to put(gi, v).
template <bool FP8, int NG, class Put>
__device__ __forceinline__ void slice_decode(Lane &st, const uint4 *mp, Put put) {
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    uint32_t v[8];
    if (FP8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t b0 = (fp8_step(st) >> 16) & 0xFFu;
        const uint32_t b1 = (fp8_step(st) >> 16) & 0xFFu;
        const uint32_t pair = b0 | (b1 << 8);
        if (j & 1)
          v[j >> 1] |= pair << 16;
        else
          v[j >> 1] = pair;
      }
    } else {
      const uint4 m = ld_nt(mp + gi * 64);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = __builtin_amdgcn_perm(bf16_step(st), dword_of(m, j >> 1), (j & 1) ? kSelHi : kSelLo);
    }
    put(gi, v);
  }
}

// Decodes NG groups of a lane's slice from a step functor (BF16: one entry
// per two weights, joined with the mantissa bytes; fp8: one code per step);
// hands each group of 16 values to put(gi, v).
template <bool FP8, int NG, class Step, class Put>
__device__ __forceinline__ void decode_groups(Step step, const uint4 (&m)[NG], Put put) {
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (FP8) {
        const uint32_t b0 = (step() >> 16) & 0xFFu;
        const uint32_t b1 = (step() >> 16) & 0xFFu;
        const uint32_t pair = b0 | (b1 << 8);
        if (j & 1)
          v[j >> 1] |= pair << 16;
        else
          v[j >> 1] = pair;
      } else {
        v[j] = __builtin_amdgcn_perm(step(), dword_of(m[gi], j >> 1), (j & 1) ? kSelHi : kSelLo);
      }
    }
    put(gi, v);
  }
}

// Persistent dequantization, on the matvec's scheme: workgroup b decodes the
// groups b, b + grid, ... with the decode table staged once per workgroup,
// the next item's code rows fetched into registers while the current item
// decodes, and items of up to kWinMax code rows decoded from a register
// window (longer ones from the wave's LDS region).  Each lane stores its
// 16-column groups straight to the output (16-byte stores when the row pitch
// allows, element stores for a ragged row end; rows past n store nothing),
// one item late: at the start of the next item, before its loads.  Stores
// count with the loads on gfx950, and stores issued after the prefetch made
// the compiler wait for them, with the prefetch, before every next item.
template <bool FP8, int NG>
__global__ __launch_bounds__(1024) void dequant_kernel(Geom g, const uint32_t *__restrict__ items,
                                                       uint8_t *__restrict__ w, int64_t ld) {
  constexpr int PR = FP8 ? 2 * NG + 4 : 2 * NG + 2;
  constexpr uint32_t kWinMax = FP8 ? 6u : 4u;
  __shared__ uint32_t s_lut[NWC_LUT_ENTRIES + (FP8 ? NWC_FP8_ESC_ENTRIES : 0)];
  extern __shared__ uint32_t s_dyn[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t region = lds_addr(s_dyn) + wave * g.region_words * 4;
  const uint32_t region_rows = g.region_words >> 6;
  const uint32_t lut = lds_addr(s_lut);
  const uint8_t *code = g.blob + g.off_code;
  const uint32_t n_groups = g.n_rowgroups * g.n_spans;
  const uint32_t first = blockIdx.x, grid = gridDim.x;
  dma_lut(g, lut, wave, g.W, lane);
  if (FP8) build_fp8_escapes(lut + NWC_LUT_BYTES, threadIdx.x, blockDim.x);
  uint32_t ahead[PR];
  fetch_code_ahead<PR>(code, items[2 * (first * g.W + wave)], items[2 * (first * g.W + wave) + 1], lane, ahead);
  // Builtin waits (the compiler's wait placement sees them, unlike inline
  // assembly, so it knows the first item's rows have arrived).
  wait_vm0();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  const int64_t esz = FP8 ? 1 : 2;
  const bool vec = (ld * esz) % 16 == 0;
  // The previous item's decoded groups, its output address and columns left.
  uint32_t out[NG][8];
  uint8_t *out_dst = w;
  int64_t out_left = 0;  // <= 0: nothing to store
  auto flush = [&] {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) put_group<FP8>(out_dst + 16 * gi * esz, out[gi], out_left - 16 * gi, vec);
  };
  for (uint32_t grp = first; grp < n_groups; grp += grid) {
    flush();
    const Place pl = place(g, grp, wave, lane);
    const uint32_t rows = items[2 * pl.item + 1];
    const uint32_t wn = rows > kWinMax ? 0u : rows < 2u ? 2u : rows;
    uint32_t cur[kWinMax];
#pragma unroll
    for (uint32_t j = 0; j < kWinMax; ++j) cur[j] = ahead[j];
    if (wn == 0) commit_code_ahead<PR>(code, items[2 * pl.item], rows, region_rows, region, lane, ahead, lane);
    uint4 m[NG];
    if (!FP8) {
      const uint4 *mp = mant_base(g, pl.item, lane);
#pragma unroll
      for (int j = 0; j < NG; ++j) m[j] = ld_nt(mp + j * 64);
    }
    {
      const bool more = grp + grid < n_groups;
      const uint32_t nx = more ? (grp + grid) * g.W + wave : pl.item;
      fetch_code_ahead<PR>(code, items[2 * nx], more ? items[2 * nx + 1] : 0u, lane, ahead);
    }
    out_dst = w + (pl.row * ld + pl.c0) * esz;
    out_left = pl.row < g.n ? g.k - pl.c0 : 0;
    auto put = [&](int gi, const uint32_t(&v)[8]) {
#pragma unroll
      for (int j = 0; j < 8; ++j) out[gi][j] = v[j];
    };
    auto run_win = [&](auto &win) {
      if constexpr (FP8)
        decode_groups<true, NG>([&] { return fp8_step_win(win, lut); }, m, put);
      else
        decode_groups<false, NG>([&] { return bf16_step_win(win, lut, g.r2s_lo, g.r2s_hi); }, m, put);
    };
    if (wn == 2) {
      Win<2> win{{cur[0], cur[1]}};
      run_win(win);
    } else if (wn == 3) {
      Win<3> win{{cur[0], cur[1], cur[2]}};
      run_win(win);
    } else if (wn == 4) {
      Win<4> win{{cur[0], cur[1], cur[2], cur[3]}};
      run_win(win);
    } else if (FP8 && wn == 5) {
      Win<5> win{{cur[0], cur[1], cur[2], cur[3], cur[kWinMax > 4 ? 4 : 0]}};
      run_win(win);
    } else if (FP8 && wn == 6) {
      Win<6> win{{cur[0], cur[1], cur[2], cur[3], cur[kWinMax > 4 ? 4 : 0], cur[kWinMax > 5 ? 5 : 0]}};
      run_win(win);
    } else {
      Lane st{region + 4 * lane, lut, 0u, g.r2s_lo, g.r2s_hi};
      if constexpr (FP8)
        decode_groups<true, NG>([&] { return fp8_step(st); }, m, put);
      else
        decode_groups<false, NG>([&] { return bf16_step(st); }, m, put);
    }
  }
  flush();
}

// ----------------------------------------------------------------- matrix-core small batches
// y_b = W x_b for a batch of up to 32 activation rows, each weight decoded
// once and multiplied on the matrix cores (v_mfma_f32_16x16x32_bf16), for
// BF16 blobs of 16 rows per work item (S = 4 slices of C = 16 or 32 columns
// per row).
//
// The matrix-core product sums over its 32-long k index in any order, so only
// A and B have to agree on which column each k stands for.  Lane l decodes the
// stream of the item's lane 4 (l % 16) + l / 16, i.e. row l % 16 and slice
// l / 16; every 8 decoded columns of its slice are then, as they come out of
// the decoder, lane l's A operand of one product (row l % 16, k = 8 (l/16) +
// i), and B is the same 8 columns of x for token l % 16: one 16-byte load.
// No tile, no LDS round trip: D (16 rows x 16 tokens, fp32; lane l holds rows
// 4 (l/16) .. +4 of token l % 16) accumulates over the item's 2C/16 products.
// Lane layouts checked on MI355X with an in-bounds probe.
//
// A workgroup of W waves (the blob's waves per group) owns one row group at a
// time, persistent over row groups; wave w takes the items (row group, span,
// w) of every span, so the waves split the columns as in the matvec.  At the
// end of a row group each wave leaves its D in its slot of one of two partial
// buffers (alternating by row group), and after one barrier the workgroup sums
// the W partials of each output in wave order (a fixed order: repeated calls
// give identical bits) and stores it.  Two buffers: a wave writes a row
// group's partials only after the barrier that ends the previous row group,
// which every thread reaches after its sums over the buffer before.
struct MfmaArgs {
  const uint8_t *mant;
  uint32_t n, k, ldx, ldy, batch, region_words, r2s_lo, r2s_hi, n_spans;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) float lds_f32;

constexpr uint32_t kMfmaPartBytes = 4 * 64 * 4;  // one wave's D for 16 tokens

template <int NG, int NH, bool RAG>
__global__ __launch_bounds__(1024) void matvec_mfma_kernel(const uint32_t *__restrict__ items,
                                                           const uint8_t *__restrict__ code,
                                                           const uint8_t *__restrict__ lut,
                                                           const uint16_t *__restrict__ x, uint32_t n_groups,
                                                           uint32_t W, const MfmaArgs a, float *__restrict__ y) {
  constexpr uint32_t C = 16 * NG;
  constexpr int PR = 2 * NG + 2;
  constexpr uint32_t kWinMax = 4;
  constexpr uint32_t kPart = NH * kMfmaPartBytes;
  __shared__ uint32_t s_lut[NWC_LUT_ENTRIES];
  extern __shared__ uint32_t s_dyn[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t src = 4u * (lane & 15u) + (lane >> 4);  // the item lane whose stream this lane decodes
  const uint32_t region = lds_addr(s_dyn) + wave * a.region_words * 4;
  const uint32_t region_rows = a.region_words >> 6;
  const uint32_t parts = lds_addr(s_dyn) + W * a.region_words * 4;  // [2][W] x kPart bytes
  const uint32_t lut_lds = lds_addr(s_lut);
  const uint32_t grid = gridDim.x, first = blockIdx.x;
  const uint32_t n_mine = (n_groups - first + grid - 1) / grid;  // grid <= n_groups
  const uint32_t total = n_mine * a.n_spans;                     // items of this wave
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void *)x, (short)0, (int)(a.batch * a.ldx * 2u), kBufWord3);
  for (uint32_t p = wave; p < NWC_LUT_BYTES / 1024; p += W) dma_1k(lut + p * 1024, lut_lds + p * 1024, 1024, lane);
  uint32_t ahead[PR];
  {
    const uint32_t it0 = first * a.n_spans * W + wave;
    fetch_code_ahead<PR>(code, items[2 * it0], items[2 * it0 + 1], src, ahead);
  }
  wait_vm0();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();

  floatx4_t acc[NH];
  uint32_t rg = first, sp = 0, parity = 0;
  for (uint32_t t = 0; t < total; ++t) {
    const uint32_t item = (rg * a.n_spans + sp) * W + wave;
    issue_priority(total, t);  // 32 rows: 132.5 -> 127.8 us per Qwen3-4B layer
    if (sp == 0) {
#pragma unroll
      for (int h = 0; h < NH; ++h) acc[h] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
    const uint32_t rows = items[2 * item + 1];
    const uint32_t wn = rows > kWinMax ? 0u : rows < 2u ? 2u : rows;
    uint32_t cur[kWinMax];
#pragma unroll
    for (uint32_t q = 0; q < kWinMax; ++q) cur[q] = ahead[q];
    if (wn == 0) commit_code_ahead<PR>(code, items[2 * item], rows, region_rows, region, lane, ahead, src);
    // This item's mantissas and activation columns, then the next item's code
    // rows (the decode waits for the code rows fetched one item earlier, the
    // products for the first two).  The activations are buffer loads over the
    // batch's rows: a token past the batch (offset past the buffer) or a
    // column block past k (offset forced past it) reads zeros, with no select
    // after the load (one would wait for the data right there).
    const uint32_t c0 = ((sp * W + wave) * 4 + (lane >> 4)) * C;  // first column of this lane's slice
    uint4 m[NG];
    {
      const uint4 *mp = (const uint4 *)(a.mant + (uint64_t)item * (64 * C)) + src;
#pragma unroll
      for (int q = 0; q < NG; ++q) m[q] = ld_nt(mp + q * 64);
    }
    u32x4_t xf[2 * NG][NH];
#pragma unroll
    for (int kb = 0; kb < 2 * NG; ++kb)
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const uint32_t tok = h * 16 + (lane & 15u), col = c0 + 8 * kb;
        const uint32_t off = col < a.k ? (tok * a.ldx + col) * 2u : 0x80000000u;
        xf[kb][h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
      }
    {
      const bool more = t + 1 < total;
      const uint32_t nx = sp + 1 < a.n_spans ? item + W : ((rg + grid) * a.n_spans) * W + wave;
      fetch_code_ahead<PR>(code, items[2 * (more ? nx : item)], more ? items[2 * nx + 1] : 0u, src, ahead);
    }
    auto put = [&](int gi, const uint32_t(&v)[8]) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const u32x4_t av = u32x4_t{v[4 * half], v[4 * half + 1], v[4 * half + 2], v[4 * half + 3]};
        // The block holding column k - 1 may run past the end of the row
        // (k not a multiple of 8): zero the activations past it.  Built only
        // where k is not a multiple of 8 (RAG): the masking ANDs cost 1-1.5 %
        // at 32 activation rows on MI355X.
        u32x4_t keep = u32x4_t{~0u, ~0u, ~0u, ~0u};
        if (RAG) {
          const uint32_t col = c0 + 8 * (2 * gi + half), valid = a.k > col ? a.k - col : 0u;
#pragma unroll
          for (int j = 0; j < 4; ++j) keep[j] = 2u * j + 1u < valid ? ~0u : 2u * j < valid ? 0xFFFFu : 0u;
        }
#pragma unroll
        for (int h = 0; h < NH; ++h)
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                          __builtin_bit_cast(bf16x8_t, RAG ? xf[2 * gi + half][h] & keep : xf[2 * gi + half][h]),
                                                          acc[h], 0, 0, 0);
      }
    };
    auto run_win = [&](auto &win) {
      decode_groups<false, NG>([&] { return bf16_step_win(win, lut_lds, a.r2s_lo, a.r2s_hi); }, m, put);
    };
    if (wn == 2) {
      Win<2> win{{cur[0], cur[1]}};
      run_win(win);
    } else if (wn == 3) {
      Win<3> win{{cur[0], cur[1], cur[2]}};
      run_win(win);
    } else if (wn == 4) {
      Win<4> win{{cur[0], cur[1], cur[2], cur[3]}};
      run_win(win);
    } else {
      Lane st{region + 4 * src, lut_lds, 0u, a.r2s_lo, a.r2s_hi};
      decode_groups<false, NG>([&] { return bf16_step(st); }, m, put);
    }
    if (sp + 1 == a.n_spans) {
      // The row group is done: partials to this wave's slot [h][i][lane],
      // one barrier, sums over the waves in wave order.
      const uint32_t buf = parts + parity * W * kPart;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *(lds_f32 *)(size_t)(buf + wave * kPart + ((h * 4 + i) * 64 + lane) * 4) = acc[h][i];
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      for (uint32_t e = threadIdx.x; e < (uint32_t)NH * 256; e += blockDim.x) {
        const uint32_t h = e >> 8, i = (e >> 6) & 3u, l = e & 63u;
        const uint32_t tok = h * 16 + (l & 15u), row = rg * 16 + (l >> 4) * 4 + i;
        if (tok < a.batch && row < a.n) {
          float sum = 0.f;
          for (uint32_t w = 0; w < W; ++w) sum += *(const lds_f32 *)(size_t)(buf + w * kPart + e * 4);
          y[(uint64_t)tok * a.ldy + row] = sum;
        }
      }
      parity ^= 1u;
      sp = 0;
      rg += grid;
    } else {
      ++sp;
    }
  }
}

// A (token, slice) unit u decodes slice u % n_sl of row ids[u / n_sl]
// (n_sl = ceil(k / C)); ids outside [0, n) give a zero row.  Thread t takes
// the units t + j * T (T threads in all, j < kGatherUnits), so the whole grid
// is resident at once.  Everything a unit needs is requested as soon as its
// address is known: the id, then its item-table entry, then at once its code
// words (a window's worth, zero past the item's rows: bounds-checked buffer
// loads over the code plane) and its mantissa chunks, for every unit of the
// thread; the decode table is copied meanwhile.  The wait for the item-table
// entries also drains the table copy, so a wave passes the start barrier with
// its code words and mantissas still in flight and decodes its first unit as
// soon as that unit's loads land (measured on MI355X, 4096 ids of 151936 x
// 2560: 10.2 us against 10.5 with every load drained before the barrier).  Each
// unit is then decoded from a register window sized to the longest item among
// the wave's lanes, as the matvec does; a wave with an item longer than the
// window copies each lane's stream to its LDS column and decodes from there.
constexpr int kGatherUnits = 2;
template <bool FP8, int NG>
__global__ __launch_bounds__(512) void gather_kernel(Geom g, const uint32_t *__restrict__ items,
                                                     const int64_t *__restrict__ ids, int64_t n_ids, uint32_t n_sl,
                                                     uint8_t *__restrict__ out) {
  constexpr uint32_t kWinMax = FP8 ? 6u : 4u;
  constexpr int U = kGatherUnits;
  __shared__ uint32_t s_lut[NWC_LUT_ENTRIES + (FP8 ? NWC_FP8_ESC_ENTRIES : 0)];
  extern __shared__ uint32_t s_dyn[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t waves = blockDim.x >> 6;
  const uint32_t lut = lds_addr(s_lut);
  dma_lut(g, lut, wave, waves, lane);
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc((void *)(g.blob + g.off_code), (short)0, (int)g.code_words4, kBufWord3);
  int64_t tok[U];
  uint32_t q[U], item[U], L[U], off[U], rows[U];
  bool live[U], valid[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t t = t0 + u * T;
    tok[u] = t / n_sl;
    q[u] = (uint32_t)(t - tok[u] * n_sl);
    live[u] = tok[u] < n_ids;
  }
  int64_t id[U];
#pragma unroll
  for (int u = 0; u < U; ++u) id[u] = live[u] ? ids[tok[u]] : 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    valid[u] = live[u] && id[u] >= 0 && id[u] < g.n;
    const int64_t row = valid[u] ? id[u] : 0;
    const uint32_t rg = (uint32_t)(row / g.R), r = (uint32_t)(row - (int64_t)rg * g.R);
    const uint32_t wq = q[u] >> g.log2S, sl = q[u] & (g.S - 1u);
    const uint32_t span = wq / g.W, wv = wq - span * g.W;
    item[u] = (rg * g.n_spans + span) * g.W + wv;
    L[u] = r * g.S + sl;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    off[u] = items[2 * item[u]];
    rows[u] = items[2 * item[u] + 1];
  }
  wait_vm0();  // the entries, and with them this wave's part of the table copy
  uint32_t w[U][kWinMax];
  uint4 m[U][NG];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (uint32_t j = 0; j < kWinMax; ++j)
      w[u][j] = __builtin_amdgcn_raw_buffer_load_b32(cr, j < rows[u] ? off[u] + j * 256 + 4 * L[u] : 0xFFFFFFF0u,
                                                     0, 0);
    if (!FP8) {
      const uint4 *mp = mant_base(g, item[u], L[u]);
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) m[u][gi] = mp[gi * 64];
    }
  }
  if (FP8) build_fp8_escapes(lut + NWC_LUT_BYTES, threadIdx.x, blockDim.x);
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  const int64_t esz = FP8 ? 1 : 2;
  const bool vec = (g.k * esz) % 16 == 0;
  const uint32_t region = lds_addr(s_dyn) + wave * g.region_words * 4;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c0 = (int64_t)q[u] * g.C;
    uint8_t *dst = out + (tok[u] * g.k + c0) * esz;
    const int64_t left = live[u] ? g.k - c0 : 0;
    const bool ok = valid[u];
    auto put = [&](int gi, const uint32_t(&v)[8]) {
      uint32_t z[8];  // an id outside [0, n): zeros (its lane decoded row 0)
#pragma unroll
      for (int i = 0; i < 8; ++i) z[i] = ok ? v[i] : 0u;
      put_group<FP8>(dst + 16 * gi * esz, z, left - 16 * gi, vec);
    };
    // Window size: the longest item among the wave's live lanes.
    const uint32_t rl = ok ? rows[u] : 0u;
    const uint32_t wn = __any(rl > kWinMax) ? 0u : __any(rl > 4) ? (__any(rl > 5) ? 6u : 5u)
                        : __any(rl > 3) ? 4u : __any(rl > 2) ? 3u : 2u;
    auto run_win = [&](auto &win) {
      if constexpr (FP8)
        decode_groups<true, NG>([&] { return fp8_step_win(win, lut); }, m[u], put);
      else
        decode_groups<false, NG>([&] { return bf16_step_win(win, lut, g.r2s_lo, g.r2s_hi); }, m[u], put);
    };
    const uint32_t(&ww)[kWinMax] = w[u];
    if (wn == 2) {
      Win<2> win{{ww[0], ww[1]}};
      run_win(win);
    } else if (wn == 3) {
      Win<3> win{{ww[0], ww[1], ww[2]}};
      run_win(win);
    } else if (wn == 4) {
      Win<4> win{{ww[0], ww[1], ww[2], ww[3]}};
      run_win(win);
    } else if (FP8 && wn == 5) {
      Win<5> win{{ww[0], ww[1], ww[2], ww[3], ww[kWinMax > 4 ? 4 : 0]}};
      run_win(win);
    } else if (FP8 && wn == 6) {
      Win<6> win{{ww[0], ww[1], ww[2], ww[3], ww[kWinMax > 4 ? 4 : 0], ww[kWinMax > 5 ? 5 : 0]}};
      run_win(win);
    } else {
      // Some lane's item is longer than the window: every lane's stream to its
      // LDS column (a lane reads and writes only its own column, in order).
      const uint32_t *src = (const uint32_t *)(g.blob + g.off_code + off[u]) + L[u];
      for (uint32_t i = 0; i < rows[u]; ++i) lds_store(region + i * 256 + 4 * lane, src[i * 64]);
      lds_store(region + rows[u] * 256 + 4 * lane, 0u);
      lds_store(region + (rows[u] + 1) * 256 + 4 * lane, 0u);
      Lane st{region + 4 * lane, lut, 0u, g.r2s_lo, g.r2s_hi};
      slice_decode<FP8, NG>(st, FP8 ? nullptr : mant_base(g, item[u], L[u]), put);
    }
  }
}

Geom make_geom(const nwc_header_t &h, const void *d_blob) {
  Geom g;
  g.blob = (const uint8_t *)d_blob;
  g.n = h.n;
  g.k = h.k;
  g.C = h.cols_per_lane;
  g.R = h.rows_per_wave;
  g.S = NWC_LANES / h.rows_per_wave;
  g.log2S = (uint32_t)__builtin_ctz(g.S);
  g.W = h.waves_per_group;
  g.n_spans = h.n_spans;
  g.n_rowgroups = h.n_rowgroups;
  g.n_items = h.n_items;
  g.region_words = (h.max_rows + NWC_GUARD_ROWS) * 64;
  g.r2s_lo = h.rank_to_sym[0] | (h.rank_to_sym[1] << 8) | (h.rank_to_sym[2] << 16) | ((uint32_t)h.rank_to_sym[3] << 24);
  g.r2s_hi = h.rank_to_sym[4] | (h.rank_to_sym[5] << 8) | (h.rank_to_sym[6] << 16) | ((uint32_t)h.rank_to_sym[7] << 24);
  g.huff = h.elem == NWC_FP8_E4M3 && h.escape_r == 0;
  g.code_words4 = (uint32_t)std::min<uint64_t>(h.code_bytes, 0xFFFFFFF0u);
  g.off_lut = h.off_lut;
  g.off_items = h.off_items;
  g.off_mant = h.off_mant;
  g.off_code = h.off_code;
  return g;
}

// Dynamic LDS of a dequant workgroup: W code regions + W*R row sums; of a
// matvec workgroup: W code regions, then per row group it decodes W*R row
// sums for each of the B activation rows.
size_t matvec_lds(const Geom &g, uint32_t groups_cap, uint32_t B = 1) {
  return (size_t)g.W * g.region_words * 4 + (size_t)groups_cap * g.W * g.R * 4 * B;
}

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Status of the launches just made.  With NWC_DEBUG set, a HIP error is also
// named on stderr.
int launched() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return NWC_OK;
  static const bool debug = getenv("NWC_DEBUG") != nullptr;
  if (debug) fprintf(stderr, "libnwc: HIP error %d (%s)\n", (int)e, hipGetErrorString(e));
  return NWC_ERR_HIP;
}

int read_header(const void *header, nwc_header_t &h) {
  if (!header) return NWC_ERR_ARG;
  memcpy(&h, header, sizeof h);
  return nwc_check_header(&h);
}

const uint32_t *item_table(const Geom &g) { return (const uint32_t *)(g.blob + g.off_items); }

// Workgroups of a launch one compute unit keeps resident at once (occupancy
// query, cached per kernel, block size and LDS), at most 25 waves per CU, and
// the number of CUs.  Measured on MI355X: the query allows 6 workgroups of 5
// waves (30 waves) per CU for the matvec, but grids sized so run slower than
// ones of 25 waves per CU.
struct Residency {
  int per_cu, cus;
  size_t lds_per_cu, lds_per_group;  // bytes: one CU's LDS, the most one workgroup may take
};
Residency resident_per_cu(const void *kernel, int block, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void *, int, size_t>, Residency> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return Residency{0, 0, 0, 0};
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(dev, kernel, block, lds);
  auto it = cache.find(key);
  if (it == cache.end()) {
    int per_cu = 0, cus = 0, lds_cu = 0, lds_wg = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, lds) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds_wg, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      return Residency{0, 0, 0, 0};
    per_cu = std::min(per_cu, std::max(1, kWavesPerCu / (block / 64)));
    it = cache.emplace(key, Residency{per_cu, cus, (size_t)lds_cu, (size_t)lds_wg}).first;
  }
  return it->second;
}

// Persistent grid: k workgroups on every compute unit, each an equal share
// (+-1) of the row groups, every grid-th one.  k is as many as fit, up to 25
// waves per compute unit: measured on MI355X, more waves than that slow every
// shape down (30 waves: +20 %), and any fewer leave the loads too few to hide
// HBM latency, even where they would give the CUs an equal number of groups
// (q 4096 x 2560: 5 workgroups 6.29 us, 4 workgroups 6.59 us).  The dynamic LDS request is padded so that no compute unit
// can take k + 1 workgroups: measured on MI355X, a grid larger than what fits
// at once leaves some workgroups to start only when others finish, on
// whichever CU frees first, so CUs end up to 25 % apart.  NWC_PERSIST=0 gives
// one workgroup per row group (for comparisons).
struct Launch {
  uint32_t grid, groups_cap;
  size_t lds;
};
Launch matvec_launch_shape(const Geom &g, const void *kernel, uint32_t B = 1, size_t static_lds = NWC_LUT_BYTES) {
  const uint32_t n_groups = g.n_rowgroups * g.n_spans;
  static const bool off = [] {
    const char *e = getenv("NWC_PERSIST");
    return e && e[0] == '0';
  }();
  const uint32_t slot = g.W * g.R * 4 * B;
  const uint32_t cap_slots = std::max<uint32_t>(1, 8192 / slot);
  Residency res{0, 0, 0, 0};
  if (!off) res = resident_per_cu(kernel, g.W * 64, matvec_lds(g, std::min<uint32_t>(cap_slots, 4), B));
  if (res.per_cu <= 0 || n_groups <= (uint32_t)res.cus) return Launch{n_groups, 1, matvec_lds(g, 1, B)};
  const uint32_t k = std::max<uint32_t>(1, (uint32_t)res.per_cu);
  uint32_t grid = std::min<uint32_t>(n_groups, k * res.cus);
  if ((n_groups + grid - 1) / grid > cap_slots) grid = (n_groups + cap_slots - 1) / cap_slots;  // LDS slots bound
  const uint32_t groups_cap = (n_groups + grid - 1) / grid;
  const size_t need = matvec_lds(g, groups_cap, B);
  // One CU's LDS / k in whole KiB less 1 KiB (k workgroups of exactly a k-th did not all fit at once
  // on MI355X), less the static decode table; at most what a workgroup may take.
  const size_t per_group = ((res.lds_per_cu / k) & ~(size_t)1023) - 1024;
  size_t share = per_group > static_lds ? per_group - static_lds : 0;
  if (res.lds_per_group > static_lds) share = std::min(share, res.lds_per_group - static_lds);
  return Launch{grid, groups_cap, std::max(need, share)};
}

// B activation rows at once (x rows ldx elements apart, y rows ldy apart);
// B > 1 only for BF16 blobs whose rows fit one workgroup.
template <bool FP8, int NG, bool SPLIT, int B, int LS>
void launch_matvec_ls(const Geom &g, hipStream_t s, const void *d_x, const float *d_scale, float *d_y, float *partial,
                      int64_t ldx, int64_t ldy) {
  const Launch L = matvec_launch_shape(g, (const void *)matvec_kernel<FP8, NG, SPLIT, B, LS>, B,
                                       NWC_LUT_BYTES + (FP8 ? NWC_FP8_ESC_ENTRIES * 4 : 0));
  MvArgs a;
  a.ldx = (uint32_t)ldx;
  a.ldy = (uint32_t)ldy;
  a.mant = g.blob + g.off_mant;
  a.n = (uint32_t)g.n;
  a.R = g.R;
  a.n_spans = g.n_spans;
  a.region_words = g.region_words;
  a.r2s_lo = g.r2s_lo;
  a.r2s_hi = g.r2s_hi;
  a.groups_cap = L.groups_cap;
  a.huff = g.huff;
  hipLaunchKernelGGL((matvec_kernel<FP8, NG, SPLIT, B, LS>), dim3(L.grid), dim3(g.W * 64), L.lds, s, item_table(g),
                     g.blob + g.off_code, g.blob + g.off_lut, (const uint16_t *)d_x, g.n_rowgroups * g.n_spans, g.W,
                     L.grid, (uint32_t)g.k, g.log2S, a, d_scale, d_y, partial);
  if (g.n_spans > 1)
    hipLaunchKernelGGL((reduce_kernel<FP8>), dim3((unsigned)((g.n * 16 + 255) / 256)), dim3(256), 0, s, partial,
                       g.n_spans, g.n, d_scale, d_y);
}

// Rows of 32 or 64 lanes (S) take kernels built for that S, whose row sums
// need no branches: for one-span, batch-1 launches of 16- and 32-column items.
// A per-launch choice rather than a branch in the kernel, whose scalar
// registers would be the most any branch needs.
template <bool FP8, int NG, bool SPLIT, int B = 1>
void launch_matvec(const Geom &g, hipStream_t s, const void *d_x, const float *d_scale, float *d_y, float *partial,
                   int64_t ldx = 0, int64_t ldy = 0) {
  if constexpr (!SPLIT && B == 1 && NG <= 2) {
    if (g.log2S == 5) return launch_matvec_ls<FP8, NG, SPLIT, B, 5>(g, s, d_x, d_scale, d_y, partial, ldx, ldy);
    if (g.log2S == 6) return launch_matvec_ls<FP8, NG, SPLIT, B, 6>(g, s, d_x, d_scale, d_y, partial, ldx, ldy);
  }
  launch_matvec_ls<FP8, NG, SPLIT, B, -1>(g, s, d_x, d_scale, d_y, partial, ldx, ldy);
}

template <bool FP8>
void launch_matvec_c(const Geom &g, hipStream_t s, const void *d_x, const float *d_scale, float *d_y,
                     float *partial) {
  if (g.n_spans > 1) {
    switch (g.C) {
      case 16: launch_matvec<FP8, 1, true>(g, s, d_x, d_scale, d_y, partial); break;
      case 32: launch_matvec<FP8, 2, true>(g, s, d_x, d_scale, d_y, partial); break;
      case 48: launch_matvec<FP8, 3, true>(g, s, d_x, d_scale, d_y, partial); break;
      default: launch_matvec<FP8, 4, true>(g, s, d_x, d_scale, d_y, partial); break;
    }
    return;
  }
  switch (g.C) {
    case 16: launch_matvec<FP8, 1, false>(g, s, d_x, d_scale, d_y, partial); break;
    case 32: launch_matvec<FP8, 2, false>(g, s, d_x, d_scale, d_y, partial); break;
    case 48: launch_matvec<FP8, 3, false>(g, s, d_x, d_scale, d_y, partial); break;
    default: launch_matvec<FP8, 4, false>(g, s, d_x, d_scale, d_y, partial); break;
  }
}

// One launch over several matrices of one work-item shape (elem, C, R, W, one
// span per row).  The persistent grid of the single-matrix launch (k
// workgroups per CU, up to 25 waves per CU) is dealt to the matrices in
// proportion to their row groups, so every workgroup gets about the same
// number of groups; workgroup order follows matrix order.  The LDS request is
// the largest any member needs, padded as for one matrix.  The kernel derives
// each matrix's row-sum slots per workgroup (ceil(groups / its workgroups))
// the same way.
template <bool FP8, int NG, int LS>
void launch_group(const Geom *g, const nwc_matvec_desc *d, int count, hipStream_t s) {
  const void *kernel = (const void *)matvec_group_kernel<FP8, NG, LS>;
  const size_t static_lds = NWC_LUT_BYTES + (FP8 ? NWC_FP8_ESC_ENTRIES * 4 : 0);
  const uint32_t W = g[0].W, slot = W * g[0].R * 4;
  const uint32_t cap_slots = std::max<uint32_t>(1, 8192 / slot);
  uint64_t total_groups = 0;
  size_t probe = 0;
  for (int m = 0; m < count; ++m) {
    total_groups += (uint64_t)g[m].n_rowgroups;
    probe = std::max(probe, matvec_lds(g[m], std::min<uint32_t>(cap_slots, 4)));
  }
  const Residency res = resident_per_cu(kernel, W * 64, probe);
  uint64_t want = total_groups;
  if (res.per_cu > 0) want = std::min<uint64_t>(total_groups, (uint64_t)res.per_cu * res.cus);
  GroupTail tail;
  memset(&tail, 0, sizeof tail);
  uint32_t grid = 0;
  size_t need = 0;
  for (int m = 0; m < count; ++m) {
    const uint32_t ng = g[m].n_rowgroups;
    uint32_t gm = (uint32_t)std::max<uint64_t>(1, (want * ng + total_groups / 2) / std::max<uint64_t>(1, total_groups));
    gm = std::min(gm, ng);
    if ((ng + gm - 1) / gm > cap_slots) gm = (ng + cap_slots - 1) / cap_slots;
    tail.begin[m] = grid;
    tail.blob[m] = g[m].blob;
    tail.x[m] = (const uint16_t *)d[m].d_x;
    tail.scale[m] = d[m].d_scale;
    tail.y[m] = d[m].d_y;
    grid += gm;
    need = std::max(need, matvec_lds(g[m], (ng + gm - 1) / gm));
  }
  tail.begin[count] = grid;
  size_t lds = need;
  if (res.per_cu > 0 && total_groups > (uint64_t)res.cus) {
    const size_t per_group = ((res.lds_per_cu / (size_t)res.per_cu) & ~(size_t)1023) - 1024;
    size_t share = per_group > static_lds ? per_group - static_lds : 0;
    if (res.lds_per_group > static_lds) share = std::min(share, res.lds_per_group - static_lds);
    lds = std::max(lds, share);
  }
  // Grid and first workgroups beyond the packed fields: the kernel reads them from the tail.
  const bool wide = grid >= (1u << 19) || (count > 1 && tail.begin[1] > 0xFFFFu) || (count > 2 && tail.begin[2] > 0xFFFFu);
  const uint32_t head = (uint32_t)count | (W << 4) | (g[0].log2S << 9) | (wide ? 1u << 12 : 0u) |
                        (wide ? 0u : grid << 13);
  const uint32_t begins = wide ? 0u : (count > 1 ? tail.begin[1] : 0u) | ((count > 2 ? tail.begin[2] : 0u) << 16);
  const uint8_t *b[3] = {tail.blob[0], count > 1 ? tail.blob[1] : tail.blob[0], count > 2 ? tail.blob[2] : tail.blob[0]};
  const uint16_t *xx[3] = {tail.x[0], count > 1 ? tail.x[1] : tail.x[0], count > 2 ? tail.x[2] : tail.x[0]};
  hipLaunchKernelGGL((matvec_group_kernel<FP8, NG, LS>), dim3(grid), dim3(W * 64), lds, s, head, begins, b[0], b[1], b[2],
                     xx[0], xx[1], xx[2], tail);
}

// Kernels built for 32 or 64 lanes per row, as for one matrix.
template <bool FP8, int NG>
void launch_group_s(const Geom *g, const nwc_matvec_desc *d, int count, hipStream_t s) {
  if constexpr (NG <= 2) {
    if (g[0].log2S == 5) return launch_group<FP8, NG, 5>(g, d, count, s);
    if (g[0].log2S == 6) return launch_group<FP8, NG, 6>(g, d, count, s);
  }
  launch_group<FP8, NG, -1>(g, d, count, s);
}

template <bool FP8>
void launch_group_c(const Geom *g, const nwc_matvec_desc *d, int count, hipStream_t s) {
  switch (g[0].C) {
    case 16: launch_group_s<FP8, 1>(g, d, count, s); break;
    case 32: launch_group_s<FP8, 2>(g, d, count, s); break;
    case 48: launch_group_s<FP8, 3>(g, d, count, s); break;
    default: launch_group_s<FP8, 4>(g, d, count, s); break;
  }
}

// Matrix-core small batch: BF16 blobs of 16 rows per work item and 16 or 32
// columns per lane; up to 32 activation rows per launch.  A persistent grid of
// workgroups of the blob's W waves, as many as fit (up to 25 waves per CU),
// each workgroup one row group at a time.
constexpr int64_t kMfmaMinBatch = 5;  // fewer rows: the VALU batch kernel
bool mfma_eligible(const nwc_header_t &h) {
  return h.elem == NWC_BF16 && h.rows_per_wave == 16 && (h.cols_per_lane == 16 || h.cols_per_lane == 32);
}

template <int NG, int NH>
void launch_mfma(const Geom &g, hipStream_t s, const void *d_x, int64_t ldx, int64_t batch, float *d_y, int64_t ldy) {
  const bool rag = (g.k & 7) != 0;
  const void *kernel = rag ? (const void *)matvec_mfma_kernel<NG, NH, true> : (const void *)matvec_mfma_kernel<NG, NH, false>;
  // Items of at most 4 code rows decode from registers; an LDS code region
  // per wave only when some item is longer.
  const uint32_t region_words = g.region_words > (4 + NWC_GUARD_ROWS) * 64 ? g.region_words : 0u;
  const size_t lds = (size_t)g.W * (region_words * 4 + 2 * NH * kMfmaPartBytes);
  const Residency res = resident_per_cu(kernel, g.W * 64, lds);
  uint32_t grid = g.n_rowgroups;
  if (res.per_cu > 0) grid = std::min<uint32_t>(grid, (uint32_t)res.per_cu * res.cus);
  MfmaArgs a;
  a.mant = g.blob + g.off_mant;
  a.n = (uint32_t)g.n;
  a.k = (uint32_t)g.k;
  a.ldx = (uint32_t)ldx;
  a.ldy = (uint32_t)ldy;
  a.batch = (uint32_t)batch;
  a.region_words = region_words;
  a.r2s_lo = g.r2s_lo;
  a.r2s_hi = g.r2s_hi;
  a.n_spans = g.n_spans;
  if (rag)
    hipLaunchKernelGGL((matvec_mfma_kernel<NG, NH, true>), dim3(grid), dim3(g.W * 64), lds, s, item_table(g),
                       g.blob + g.off_code, g.blob + g.off_lut, (const uint16_t *)d_x, g.n_rowgroups, g.W, a, d_y);
  else
    hipLaunchKernelGGL((matvec_mfma_kernel<NG, NH, false>), dim3(grid), dim3(g.W * 64), lds, s, item_table(g),
                       g.blob + g.off_code, g.blob + g.off_lut, (const uint16_t *)d_x, g.n_rowgroups, g.W, a, d_y);
}

void launch_mfma_c(const Geom &g, hipStream_t s, const uint16_t *x, int64_t ldx, int64_t batch, float *y,
                   int64_t ldy) {
  for (int64_t b = 0; b < batch; b += 32) {
    const int64_t nb = std::min<int64_t>(32, batch - b);
    const uint16_t *xb = x + b * ldx;
    float *yb = y + b * ldy;
    if (g.C == 16) {
      if (nb > 16) launch_mfma<1, 2>(g, s, xb, ldx, nb, yb, ldy);
      else launch_mfma<1, 1>(g, s, xb, ldx, nb, yb, ldy);
    } else {
      if (nb > 16) launch_mfma<2, 2>(g, s, xb, ldx, nb, yb, ldy);
      else launch_mfma<2, 1>(g, s, xb, ldx, nb, yb, ldy);
    }
  }
}

// B = 2 or 4 activation rows of a BF16 blob with one span per row and 16 or
// 32 columns per lane (wider items would not keep B rows of activations in
// registers).
template <int B>
void launch_matvec_rows(const Geom &g, hipStream_t s, const void *d_x, int64_t ldx, float *d_y, int64_t ldy) {
  if (g.C == 16)
    launch_matvec<false, 1, false, B>(g, s, d_x, nullptr, d_y, nullptr, ldx, ldy);
  else
    launch_matvec<false, 2, false, B>(g, s, d_x, nullptr, d_y, nullptr, ldx, ldy);
}

// Persistent grid as for the matvec (k workgroups per CU, up to 25 waves, the
// LDS request padded so that no CU takes k + 1); a workgroup's LDS is its
// waves' code regions only.
template <bool FP8, int NG>
void launch_dequant(const Geom &g, hipStream_t s, void *d_w, int64_t ld) {
  const void *kernel = (const void *)dequant_kernel<FP8, NG>;
  const uint32_t n_groups = g.n_rowgroups * g.n_spans;
  const size_t regions = (size_t)g.W * g.region_words * 4;
  const size_t static_lds = NWC_LUT_BYTES + (FP8 ? NWC_FP8_ESC_ENTRIES * 4 : 0);
  const Residency res = resident_per_cu(kernel, g.W * 64, regions);
  uint32_t grid = n_groups;
  size_t lds = regions;
  if (res.per_cu > 0 && n_groups > (uint32_t)res.cus) {
    const uint32_t k = (uint32_t)res.per_cu;
    grid = std::min<uint32_t>(n_groups, k * res.cus);
    const size_t per_group = ((res.lds_per_cu / k) & ~(size_t)1023) - 1024;
    size_t share = per_group > static_lds ? per_group - static_lds : 0;
    if (res.lds_per_group > static_lds) share = std::min(share, res.lds_per_group - static_lds);
    lds = std::max(lds, share);
  }
  hipLaunchKernelGGL((dequant_kernel<FP8, NG>), dim3(grid), dim3(g.W * 64), lds, s, g, item_table(g), (uint8_t *)d_w,
                     ld);
}

template <bool FP8>
void launch_dequant_c(const Geom &g, hipStream_t s, void *d_w, int64_t ld) {
  switch (g.C) {
    case 16: launch_dequant<FP8, 1>(g, s, d_w, ld); break;
    case 32: launch_dequant<FP8, 2>(g, s, d_w, ld); break;
    case 48: launch_dequant<FP8, 3>(g, s, d_w, ld); break;
    default: launch_dequant<FP8, 4>(g, s, d_w, ld); break;
  }
}

// Gather workgroups hold as many waves (up to 16) as their code columns fit
// the LDS the matvec workgroup may use.
template <bool FP8, int NG>
void launch_gather(const Geom &g, hipStream_t s, const int64_t *d_ids, int64_t n_ids, void *d_out) {
  const uint32_t n_sl = (uint32_t)((g.k + g.C - 1) / g.C);
  const int64_t units = n_ids * n_sl;
  // Workgroups of 4 waves (or as many as the LDS regions allow), each thread
  // kGatherUnits units: the grid of a 4096-id gather is resident at once.
  // Measured on MI355X (4096 ids of 151936 x 2560): 4 waves 10.4 us, 8 waves
  // 10.7, 16 waves 11.4, 2 waves 12.2.
  const uint32_t fit = (uint32_t)((NWC_LDS_BUDGET - NWC_LUT_BYTES) / (g.region_words * 4));
  const uint32_t waves = fit < 1 ? 1 : fit > 4 ? 4 : fit;
  const uint32_t tpb = waves * 64;
  const int64_t threads = (units + kGatherUnits - 1) / kGatherUnits;
  hipLaunchKernelGGL((gather_kernel<FP8, NG>), dim3((unsigned)((threads + tpb - 1) / tpb)), dim3(tpb),
                     (size_t)waves * g.region_words * 4, s, g, item_table(g), d_ids, n_ids, n_sl, (uint8_t *)d_out);
}

template <bool FP8>
void launch_gather_c(const Geom &g, hipStream_t s, const int64_t *d_ids, int64_t n_ids, void *d_out) {
  switch (g.C) {
    case 16: launch_gather<FP8, 1>(g, s, d_ids, n_ids, d_out); break;
    case 32: launch_gather<FP8, 2>(g, s, d_ids, n_ids, d_out); break;
    case 48: launch_gather<FP8, 3>(g, s, d_ids, n_ids, d_out); break;
    default: launch_gather<FP8, 4>(g, s, d_ids, n_ids, d_out); break;
  }
}

// Plain streaming read (the achievable-bandwidth reference for the matvec, not
// part of the method): every 16-byte chunk of the buffer is loaded once by a
// grid-stride loop; what is read is XOR-folded and stored only if it equals a
// value it practically never has, so no load can be dropped.  Measured on
// MI355X, one non-temporal load per iteration and 8 workgroups of 256 per CU
// read fastest (1 GiB: 7.15 TB/s; default cache policy 6.54 TB/s; two or four
// loads per iteration 5.3-6.0 TB/s).
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ p, uint64_t n16,
                                                          uint32_t *__restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const uint4 v = ld_nt(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Scratch of nwc_matvec_noalloc: the fp32 span partials of matrices whose
// rows span several workgroups, in a file-scope device array (each GPU the
// library runs on holds its own copy until the process ends).  In host code
// `nwc_scratch` only names the array; its device address, which differs per
// GPU, comes from hipGetSymbolAddress, taken once per device with that device
// current and kept in scratch_ptr[].
__device__ __align__(256) float nwc_scratch[NWC_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;

// Device address of this GPU's nwc_scratch (nullptr and NWC_ERR_HIP on failure).
int scratch_for_current_device(float **out) {
  static std::mutex mu;
  static float *ptr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NWC_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(nwc_scratch)) != hipSuccess || !p) return NWC_ERR_HIP;
    ptr[dev] = (float *)p;
  }
  *out = ptr[dev];
  return NWC_OK;
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
  if (fp8)
    launch_matvec_c<true>(g, s, d_x, d_scale, d_y, partial);
  else
    launch_matvec_c<false>(g, s, d_x, d_scale, d_y, partial);
  return launched();
}

int nwc_matvec_noalloc(const void *header, const void *d_blob, const void *d_x, const float *d_scale, float *d_y,
                       void *stream) {
  nwc_header_t h;
  int st = read_header(header, h);
  if (st != NWC_OK) return st;
  int64_t need = 0;
  if ((st = nwc_workspace_size(header, &need)) != NWC_OK) return st;
  if (need > (int64_t)NWC_NOALLOC_SCRATCH_BYTES) return NWC_ERR_CAPACITY;
  if (!d_blob || !d_x || !d_y || !aligned(d_blob, 16) || !aligned(d_x, 16) || !aligned(d_y, 4)) return NWC_ERR_ARG;
  const bool fp8 = h.elem == NWC_FP8_E4M3;
  if (fp8 != (d_scale != nullptr) || (d_scale && !aligned(d_scale, 4))) return NWC_ERR_ARG;
  float *partial = nullptr;
  if (need > 0 && (st = scratch_for_current_device(&partial)) != NWC_OK) return st;
  const Geom g = make_geom(h, d_blob);
  hipStream_t s = (hipStream_t)stream;
  if (fp8)
    launch_matvec_c<true>(g, s, d_x, d_scale, d_y, partial);
  else
    launch_matvec_c<false>(g, s, d_x, d_scale, d_y, partial);
  return launched();
}

int nwc_matvec_group(const nwc_matvec_desc *mats, int count, void *stream) {
  if (count < 0 || count > NWC_GROUP_MAX) return NWC_ERR_SHAPE;
  if (count == 0) return NWC_OK;
  if (!mats) return NWC_ERR_ARG;
  // Every member checked before anything is enqueued.
  nwc_header_t h[NWC_GROUP_MAX];
  Geom g[NWC_GROUP_MAX];
  for (int m = 0; m < count; ++m) {
    const nwc_matvec_desc &d = mats[m];
    int st = read_header(d.header, h[m]);
    if (st != NWC_OK) return st;
    if (!d.d_blob || !d.d_x || !d.d_y || !aligned(d.d_blob, 16) || !aligned(d.d_x, 16) || !aligned(d.d_y, 4))
      return NWC_ERR_ARG;
    const bool fp8 = h[m].elem == NWC_FP8_E4M3;
    if (fp8 != (d.d_scale != nullptr) || (d.d_scale && !aligned(d.d_scale, 4))) return NWC_ERR_ARG;
    if (h[m].n_spans != 1) return NWC_ERR_UNSUPPORTED;
    g[m] = make_geom(h[m], d.d_blob);
  }
  // One launch per work-item shape, members in their order of appearance.
  hipStream_t s = (hipStream_t)stream;
  bool done[NWC_GROUP_MAX] = {};
  for (int m = 0; m < count; ++m) {
    if (done[m]) continue;
    Geom gs[NWC_GROUP_MAX];
    nwc_matvec_desc ds[NWC_GROUP_MAX];
    int c = 0;
    for (int j = m; j < count; ++j) {
      if (done[j] || h[j].elem != h[m].elem || g[j].C != g[m].C || g[j].R != g[m].R || g[j].W != g[m].W) continue;
      done[j] = true;
      gs[c] = g[j];
      ds[c] = mats[j];
      ++c;
    }
    // Members in ascending order of row groups (stable).  Measured on MI355X
    // (Qwen3-4B layers, medians of 5): q,k,v with q first 8.27 us, with q
    // last 7.53 us.  Each output is the same in any order.
    for (int i = 1; i < c; ++i)
      for (int j = i; j > 0 && gs[j].n_rowgroups < gs[j - 1].n_rowgroups; --j) {
        std::swap(gs[j], gs[j - 1]);
        std::swap(ds[j], ds[j - 1]);
      }
    if (h[m].elem == NWC_FP8_E4M3)
      launch_group_c<true>(gs, ds, c, s);
    else
      launch_group_c<false>(gs, ds, c, s);
  }
  return launched();
}

int nwc_matvec_batch(const void *header, const void *d_blob, const void *d_x, int64_t ldx, int64_t batch,
                     const float *d_scale, float *d_y, int64_t ldy, void *d_ws, int64_t ws_bytes, void *stream) {
  nwc_header_t h;
  int st = read_header(header, h);
  if (st != NWC_OK) return st;
  if (batch < 0 || ldx < h.k || ldy < h.n || ldx % 8 != 0 || ldx >= ((int64_t)1 << 31) || ldy >= ((int64_t)1 << 31))
    return NWC_ERR_SHAPE;
  if (batch == 0) return NWC_OK;
  const bool fp8 = h.elem == NWC_FP8_E4M3;
  if (!d_blob || !d_x || !d_y || !aligned(d_blob, 16) || !aligned(d_x, 16) || !aligned(d_y, 4)) return NWC_ERR_ARG;
  if (fp8 != (d_scale != nullptr) || (d_scale && !aligned(d_scale, 4))) return NWC_ERR_ARG;
  const uint16_t *x = (const uint16_t *)d_x;
  if (mfma_eligible(h) && batch >= kMfmaMinBatch && ldx < ((int64_t)1 << 25)) {  // matrix cores, 32 rows per decode
    launch_mfma_c(make_geom(h, d_blob), (hipStream_t)stream, x, ldx, batch, d_y, ldy);
    return launched();
  }
  if (fp8 || h.n_spans > 1 || h.cols_per_lane > 32) {  // one activation row at a time
    for (int64_t b = 0; b < batch; ++b)
      if ((st = nwc_matvec(header, d_blob, x + b * ldx, d_scale, d_y + b * ldy, d_ws, ws_bytes, stream)) != NWC_OK)
        return st;
    return NWC_OK;
  }
  const Geom g = make_geom(h, d_blob);
  hipStream_t s = (hipStream_t)stream;
  int64_t b = 0;
  for (; batch - b >= 4; b += 4) launch_matvec_rows<4>(g, s, x + b * ldx, ldx, d_y + b * ldy, ldy);
  if (batch - b >= 2) {
    launch_matvec_rows<2>(g, s, x + b * ldx, ldx, d_y + b * ldy, ldy);
    b += 2;
  }
  if (b < batch) launch_matvec_c<false>(g, s, x + b * ldx, nullptr, d_y + b * ldy, nullptr);
  return launched();
}

int nwc_dequant(const void *header, const void *d_blob, void *d_w, int64_t ld, void *stream) {
  nwc_header_t h;
  int st = read_header(header, h);
  if (st != NWC_OK) return st;
  if (!d_blob || !d_w || !aligned(d_blob, 16) || !aligned(d_w, 16)) return NWC_ERR_ARG;
  if (ld < h.k) return NWC_ERR_SHAPE;
  const Geom g = make_geom(h, d_blob);
  hipStream_t s = (hipStream_t)stream;
  if (h.elem == NWC_FP8_E4M3)
    launch_dequant_c<true>(g, s, d_w, ld);
  else
    launch_dequant_c<false>(g, s, d_w, ld);
  return launched();
}

int nwc_gather(const void *header, const void *d_blob, const int64_t *d_ids, int64_t n_ids, void *d_out,
               void *stream) {
  nwc_header_t h;
  int st = read_header(header, h);
  if (st != NWC_OK) return st;
  const int64_t n_sl = (h.k + h.cols_per_lane - 1) / h.cols_per_lane;
  if (n_ids < 0 || n_ids * n_sl > ((int64_t)1 << 40)) return NWC_ERR_SHAPE;
  if (n_ids == 0) return NWC_OK;
  if (!d_blob || !d_ids || !d_out || !aligned(d_blob, 16) || !aligned(d_ids, 8) || !aligned(d_out, 16))
    return NWC_ERR_ARG;
  const Geom g = make_geom(h, d_blob);
  hipStream_t s = (hipStream_t)stream;
  if (h.elem == NWC_FP8_E4M3)
    launch_gather_c<true>(g, s, d_ids, n_ids, d_out);
  else
    launch_gather_c<false>(g, s, d_ids, n_ids, d_out);
  return launched();
}

int nwc_stream_read(const void *d_buf, int64_t bytes, uint32_t *d_sink, void *stream) {
  if (!d_buf || !d_sink || !aligned(d_buf, 16) || !aligned(d_sink, 4)) return NWC_ERR_ARG;
  if (bytes < 0 || bytes % 16) return NWC_ERR_SHAPE;
  if (bytes == 0) return NWC_OK;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return NWC_ERR_HIP;
  const uint64_t n16 = (uint64_t)bytes / 16;
  const uint64_t want = (n16 + 255) / 256;  // workgroups that each get at least one load per thread
  const unsigned grid = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(want, (uint64_t)cus * 8));
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const uint4 *)d_buf, n16,
                     d_sink);
  return launched();
}

}  // extern "C"
