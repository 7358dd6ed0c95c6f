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
//   items      8 B per work item: {u32 code byte offset, u32 code rows}
//   mant       BF16 only: raw mantissa bytes, 64*C bytes per item
//   code       per item: code_rows x 64 lane columns of u32
//
// Geometry.  A work item is what one wave decodes: R rows (R = rows_per_wave,
// a power of two) times S = 64/R slices per row, a slice being C consecutive
// columns (C = cols_per_lane, a multiple of 16).  Lane L of an item holds row
// L / S of its row group and slice L % S, so the S lanes of a row are
// adjacent.  A row's slices are numbered q = 0, 1, ... (columns [qC, qC+C)).
// A group of W consecutive items (W = waves_per_group, one workgroup) covers
// S*W consecutive slices of the same R rows; n_spans groups cover a whole row
// group (one in every shape with K <= 16*S*C).
//   item = (row_group * n_spans + span) * W + wave
//   lane L: row = row_group*R + L/S, slice q = (span*W + wave)*S + L%S
//
// Fillers.  Columns at or past K and rows at or past N are fillers: zero code
// bits, which decode as rank 0 with sign 0, and zero mantissa bytes (the
// Huffman variant writes byte 0x00's codeword instead).  A filler
// therefore decodes to a finite value (BF16 exponent field 2*symbol <= 254;
// fp8 mantissa 0 is never NaN) and adds exactly zero against the zero
// activation the kernel uses past column K.
//
// Code plane of an item: lane L owns column L of a (code_rows x 64) u32 array,
// i.e. its stream's word w lives at u32 index w*64 + L.  A lane's stream starts
// with 2 zero bits, then the codes of its C columns (fillers included) in
// column order, bits least-significant first; code_rows covers the longest
// lane, shorter lanes are zero-padded.  Decoders keep two zero rows after the
// item's rows so a 64-bit read at the last code stays defined.
//
// Mantissa plane of an item (BF16): lane L's mantissa bytes in column order,
// in 16-byte chunks; chunk j of lane L at byte (j*64 + L)*16 of the item's
// 64*C-byte block, so a wave's load of chunk j is one contiguous KiB.
//
// Decode table (BF16): entry for peek p (12 stream bits, first bit = bit 0):
//   two complete codes A, B within the 12 bits:
//     bits 0..7 bits used, 8..15 high byte of A, 16..23 high byte of B, 31 = 0
//   otherwise (escape or a longer pair): bit 31 = 1, rest 0.
// Decode table (fp8): one code per peek:
//   bits 0..15 the value as BF16, 16..23 the fp8 byte, 24..30 bits used,
//   31 = 1 if the code is an escape (longer than 12 bits).
//
// Coder variant (escape_r == 0, fp8 only): a length-limited canonical Huffman
// code over whole fp8 bytes.  Codeword lengths (at most NWC_HUFF_MAX_LEN = 12
// bits, optimal for the matrix's byte histogram, found by package-merge) are
// stored as nibbles in rank_to_sym; codewords are canonical (bytes in order of
// (length, value); the first is all zeros; each next is the previous plus one,
// shifted left by the growth in length) and written most significant bit
// first.  Byte 0x00 always has a codeword: it is the filler of this variant
// (fillers are written as its codeword, so they decode to +0).  Every
// codeword fits the 12-bit peek, so the fp8 decode table above decodes every
// code and has no escapes.
#pragma once
#include <stdint.h>

#define NWC_MAGIC 0x3143574Eu /* "NWC1" */
#define NWC_FORMAT_VERSION 4u
#define NWC_HEADER_BYTES 256
#define NWC_LANES 64
#define NWC_LUT_ENTRIES 4096
#define NWC_LUT_BYTES (NWC_LUT_ENTRIES * 4)
#define NWC_ESCAPE_R 8
#define NWC_HUFF_MAX_LEN 12 /* longest Huffman codeword: the decode table's peek */
#define NWC_LEAD_BITS 2
#define NWC_MAX_COLS 64     /* cols_per_lane: multiple of 16 in [16, 64] */
#define NWC_MAX_WAVES 16    /* waves per workgroup (1024 threads) */
#define NWC_ROWS_CAP 40     /* longest lane stream: 2 + 16*64 bits < 33 words */
#define NWC_GUARD_ROWS 2
#define NWC_LDS_BUDGET (64 * 1024) /* decoder LDS per workgroup the encoder plans for */

#ifdef __cplusplus
extern "C" {
#endif

typedef struct nwc_header_t {
  uint32_t magic;
  uint32_t version;
  uint32_t elem;             /* 0 = BF16, 1 = fp8 e4m3fn */
  uint32_t header_bytes;
  int64_t n;                 /* rows (output features) */
  int64_t k;                 /* columns (input features) */
  uint32_t cols_per_lane;    /* C */
  uint32_t rows_per_wave;    /* R, power of two in [1, 64] */
  uint32_t waves_per_group;  /* W, 1..16 */
  uint32_t n_spans;          /* workgroups per row group */
  uint32_t n_rowgroups;      /* ceil(n / R) */
  uint32_t n_items;          /* n_rowgroups * n_spans * W */
  uint32_t max_rows;         /* largest code_rows of any item */
  uint32_t escape_r;         /* 8: unary rank code; 0: Huffman over fp8 bytes */
  uint64_t coded_bits;       /* code bits of the real weights (+ 8 per BF16 weight) */
  uint64_t off_lut, off_items, off_mant, off_code;
  uint64_t total_bytes;
  uint64_t code_bytes, mant_bytes;
  uint8_t rank_to_sym[128];  /* 128 BF16 symbols, or 16 fp8 exponent fields;
                                Huffman: codeword length of byte b in nibble b
                                (byte b/2, low nibble for even b), 0 = none */
} nwc_header_t;

#ifdef __cplusplus
static_assert(sizeof(nwc_header_t) == NWC_HEADER_BYTES, "header must be 256 bytes");
}
#endif
