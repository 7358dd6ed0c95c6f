// Blob format of the compressed matrices (host encoder <-> gfx950 kernels).
//
// The code is the one on the "neural-weight-compression 0.9.0" PyPI page,
// "How it works": each BF16 weight is split into a raw mantissa byte (the low
// byte) and an exponent/sign byte (the high byte); the 7-bit exponent symbol is
// ranked by frequency per matrix and written as a unary rank code followed by
// the raw sign bit, with an escape carrying the raw symbol for rare values.
// Bit-level choices (ones-then-zero unary, least-significant-bit-first
// streams, escape after 8 ranks) are readings of that page.  The stream layout
// below is this library's own, chosen for 64-lane wavefronts.
//
// Layout (little endian, every section 256-byte aligned):
//   header     256 B    nwc_header_t
//   lut        16 KiB   4096 x u32 decode table indexed by a 12-bit peek
//   items      8 B per item: {u32 code_offset, u32 code_rows}
//   mant       BF16 only: raw mantissa bytes
//   code       per item: code_rows x 64 lane columns of u32
//
// Work item = 64 matrix rows (one per lane of a wave) x cols_per_item columns.
// Items are numbered item = rowblock * n_kspans + kspan.
//
// Code plane of an item: lane L owns column L of a (code_rows x 64) u32 array,
// i.e. its stream's word w lives at u32 index w*64 + L.  A lane's stream starts
// with 2 zero bits, then the codes of its row's weights in column order, bits
// least-significant first.  Columns are zero-padded to the item's longest
// stream.  Rows past N have empty (all-zero) streams.
//
// Mantissa plane of an item (BF16): lane L's mantissa bytes in column order,
// in 16-byte chunks; chunk j of lane L at byte (j*64 + L)*16 of the item's
// region.  Item (rb, ks) region starts at rb*64*k_pad + 64*ks*cols_per_item,
// where k_pad sums each kspan's column count rounded up to 16.
//
// Decode table (BF16): entry for peek p (12 stream bits, first bit = bit 0):
//   two complete codes A, B within the 12 bits:
//     bits 0..7 high byte of A, 8..15 high byte of B, 16..23 bits used, 31 = 0
//   otherwise (escape or a longer pair): bit 31 = 1, rest 0.
// Decode table (fp8): one code per peek:
//   bits 0..15 the value as BF16, 16..23 the fp8 byte, 24..30 bits used,
//   31 = 1 if the code is an escape (longer than 12 bits).
#pragma once
#include <stdint.h>

#define NWC_MAGIC 0x3143574Eu /* "NWC1" */
#define NWC_FORMAT_VERSION 1u
#define NWC_HEADER_BYTES 256
#define NWC_LANES 64
#define NWC_LUT_ENTRIES 4096
#define NWC_LUT_BYTES (NWC_LUT_ENTRIES * 4)
#define NWC_ESCAPE_R 8
#define NWC_LEAD_BITS 2
#define NWC_ROWS_CAP 40
#define NWC_MAX_COLS 256
#define NWC_MIN_COLS 64
#define NWC_GUARD_ROWS 2

#ifdef __cplusplus
extern "C" {
#endif

typedef struct nwc_header_t {
  uint32_t magic;
  uint32_t version;
  uint32_t elem;           /* 0 = BF16, 1 = fp8 e4m3fn */
  uint32_t header_bytes;
  int64_t n;               /* rows (output features) */
  int64_t k;               /* columns (input features) */
  uint32_t cols_per_item;  /* multiple of 16, 16..256 */
  uint32_t n_rowblocks;    /* ceil(n / 64) */
  uint32_t n_kspans;       /* ceil(k / cols_per_item) */
  uint32_t n_items;        /* n_rowblocks * n_kspans */
  uint32_t max_rows;       /* largest code_rows of any item */
  uint32_t escape_r;       /* 8 */
  uint32_t last_cols;      /* columns of the last kspan */
  uint32_t k_pad;          /* sum over kspans of round_up(cols, 16) */
  uint64_t coded_bits;     /* code bits of the real weights (+ 8 per BF16 weight) */
  uint64_t off_lut, off_items, off_mant, off_code;
  uint64_t total_bytes;
  uint64_t code_bytes, mant_bytes;
  uint8_t rank_to_sym[128]; /* 128 BF16 symbols, or 16 fp8 exponent fields */
} nwc_header_t;

#ifdef __cplusplus
static_assert(sizeof(nwc_header_t) == NWC_HEADER_BYTES, "header must be 256 bytes");
}
#endif
