/*
 * nwc_oracle.c -- the CPU oracle's codec and float64 matvec in plain C, for
 * full-size workloads (billions of weights) that the numpy oracle would take
 * hours over.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this file's library.  It shares no code,
 * header, table or constant with the product library (decode_matvec_amd/) and
 * includes nothing from it.
 *
 * What it computes is what oracle/nwc_ref.py computes, written again as plain
 * scalar C: one bit stream per matrix row, codes appended in column order,
 * stream bit p stored in bit (p mod 64) of 64-bit word p / 64 (least
 * significant bit first).  Every function cites the passage it follows:
 *  - byte split and ranking: "neural-weight-compression 0.9.0" PyPI page,
 *    "How it works", first and second bullets (mantissa byte raw,
 *    exponent/sign byte ranked by frequency per matrix, unary rank code plus a
 *    raw sign bit, escape for rare values);
 *  - fp8: "Qwen3-4B-NWC-fp8" model card, summary and "How it was made"
 *    (weight-only e4m3 with a per-output-channel scale applied after the row
 *    sum, fp8 bytes coded whole and recovered bit for bit).
 * Readings where the pages are silent (escape after eight ranks, ones-then-zero
 * unary, least-significant-bit-first order, ties ranked by ascending symbol)
 * are the ones oracle/nwc_ref.py states, and the tests check that both oracles
 * write identical bits.
 *
 * Error behaviour: functions return a negative value on a capacity overflow or
 * on a stream that does not decode to its recorded length; nothing aborts.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ESCAPE_RANKS 8 /* ranks 0..7 get unary codes; the rest escape */

/* ---------------------------------------------------------------- bit streams */
static void put_bit(uint64_t *s, int64_t p, unsigned b) {
  if (b) s[p >> 6] |= (uint64_t)1 << (p & 63);
}

static unsigned get_bit(const uint64_t *s, int64_t p) { return (unsigned)(s[p >> 6] >> (p & 63)) & 1u; }

/* ---------------------------------------------------------------- ranking */
/* Frequency rank table (PyPI page, "How it works", second bullet: "ranked by
 * frequency"): rank 0 is the most frequent symbol; equal counts are ordered by
 * ascending symbol.  Every symbol of the alphabet gets a rank. */
void nwc_oracle_rank_table(const uint64_t *counts, int alphabet, uint8_t *rank_to_sym, uint8_t *sym_to_rank) {
  unsigned char used[256];
  memset(used, 0, sizeof used);
  for (int r = 0; r < alphabet; ++r) {
    int best = -1;
    for (int s = 0; s < alphabet; ++s)
      if (!used[s] && (best < 0 || counts[s] > counts[best])) best = s;
    used[best] = 1;
    rank_to_sym[r] = (uint8_t)best;
    sym_to_rank[best] = (uint8_t)r;
  }
}

/* ---------------------------------------------------------------- BF16 */
/* Byte planes (PyPI page, "How it works", first bullet): the high byte of a
 * BF16 weight is the sign and the 7-bit exponent symbol e = (u >> 8) & 0x7F;
 * the low byte is the raw mantissa byte.  Histogram of e over the matrix. */
void nwc_oracle_bf16_histogram(const uint16_t *w, int64_t n, int64_t k, int64_t ld, uint64_t *counts128) {
  memset(counts128, 0, 128 * sizeof(uint64_t));
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < k; ++j) counts128[(w[i * ld + j] >> 8) & 0x7F]++;
}

/* Histogram of the whole high byte (sign included), for its entropy. */
void nwc_oracle_bf16_hi_histogram(const uint16_t *w, int64_t n, int64_t k, int64_t ld, uint64_t *counts256) {
  memset(counts256, 0, 256 * sizeof(uint64_t));
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < k; ++j) counts256[w[i * ld + j] >> 8]++;
}

/* One codeword at stream bit p; returns the bit after it.  Rank r < 8: r
 * one-bits, a zero-bit, the sign.  Rank >= 8 (escape): eight one-bits, the
 * sign, then the 7 symbol bits least significant first. */
static int64_t put_code_bf16(uint64_t *s, int64_t p, unsigned rank, unsigned sign, unsigned sym) {
  if (rank < ESCAPE_RANKS) {
    for (unsigned i = 0; i < rank; ++i) put_bit(s, p++, 1);
    put_bit(s, p++, 0);
    put_bit(s, p++, sign);
  } else {
    for (unsigned i = 0; i < ESCAPE_RANKS; ++i) put_bit(s, p++, 1);
    put_bit(s, p++, sign);
    for (unsigned i = 0; i < 7; ++i) put_bit(s, p++, (sym >> i) & 1u);
  }
  return p;
}

/* Encodes rows of a BF16 matrix (uint16 patterns, row pitch ld) with the given
 * symbol ranks: row i's stream starts at bit row_start[i] of `stream` and ends
 * at row_start[i + 1] (n + 1 entries written).  stream_words 64-bit words are
 * available; they are cleared first.  Returns the total code bits, or -1 if
 * the stream does not fit. */
int64_t nwc_oracle_bf16_encode(const uint16_t *w, int64_t n, int64_t k, int64_t ld, const uint8_t *sym_to_rank,
                               uint64_t *stream, int64_t stream_words, int64_t *row_start) {
  memset(stream, 0, (size_t)stream_words * sizeof(uint64_t));
  const int64_t cap = stream_words * 64;
  int64_t p = 0;
  for (int64_t i = 0; i < n; ++i) {
    row_start[i] = p;
    for (int64_t j = 0; j < k; ++j) {
      const unsigned u = w[i * ld + j];
      const unsigned sign = u >> 15, sym = (u >> 8) & 0x7F;
      if (p + 16 > cap) return -1;
      p = put_code_bf16(stream, p, sym_to_rank[sym], sign, sym);
    }
  }
  row_start[n] = p;
  return p;
}

/* Decodes the rows written by nwc_oracle_bf16_encode: code at the stream
 * position, then the raw mantissa byte mant[i * ldm + j]; the weight is
 * sign << 15 | symbol << 8 | mantissa.  A code's ones are counted up to eight
 * (eight ones = escape).  Returns 0, or -1 if a row's codes do not end exactly
 * at the next row's start. */
int nwc_oracle_bf16_decode(const uint64_t *stream, const int64_t *row_start, int64_t n, int64_t k,
                           const uint8_t *rank_to_sym, const uint8_t *mant, int64_t ldm, uint16_t *out, int64_t ldo) {
  for (int64_t i = 0; i < n; ++i) {
    int64_t p = row_start[i];
    const int64_t end = row_start[i + 1];
    for (int64_t j = 0; j < k; ++j) {
      if (p + 2 > end) return -1;
      unsigned ones = 0;
      while (ones < ESCAPE_RANKS && p < end && get_bit(stream, p)) {
        ++ones;
        ++p;
      }
      unsigned sign, sym;
      if (ones < ESCAPE_RANKS) {
        ++p; /* the terminating zero */
        if (p >= end) return -1;
        sign = get_bit(stream, p++);
        sym = rank_to_sym[ones];
      } else {
        if (p + 8 > end) return -1;
        sign = get_bit(stream, p++);
        sym = 0;
        for (unsigned b = 0; b < 7; ++b) sym |= get_bit(stream, p++) << b;
      }
      out[i * ldo + j] = (uint16_t)((sign << 15) | (sym << 8) | mant[i * ldm + j]);
    }
    if (p != end) return -1;
  }
  return 0;
}

/* Exact value of a BF16 pattern: the pattern is the top half of an fp32. */
static double bf16_value(uint16_t u) {
  const uint32_t b = (uint32_t)u << 16;
  float f;
  memcpy(&f, &b, sizeof f);
  return (double)f;
}

/* Batch-1 matvec in float64 (PyPI page, "How it works", fused-kernel bullet:
 * row sums of weight times activation): y_i = sum_j w_ij x_j in column order,
 * and a_i = sum_j |w_ij x_j|, which bounds the rounding of any summation order. */
void nwc_oracle_bf16_matvec(const uint16_t *w, int64_t n, int64_t k, int64_t ld, const uint16_t *x, double *y,
                            double *a) {
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0, t = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      const double p = bf16_value(w[i * ld + j]) * bf16_value(x[j]);
      s += p;
      t += fabs(p);
    }
    y[i] = s;
    a[i] = t;
  }
}

/* ---------------------------------------------------------------- fp8 e4m3fn */
/* Model card "Qwen3-4B-NWC-fp8": the fp8 byte b = sign << 7 | E << 3 | M is
 * coded whole.  Reading: the 4-bit exponent field E is the ranked symbol;
 * rank r < 8 is r one-bits, a zero-bit, the sign, then M (3 bits, least
 * significant first); an escape is eight one-bits, the sign, E (4 bits), M. */
void nwc_oracle_fp8_histogram(const uint8_t *q, int64_t n, int64_t k, int64_t ld, uint64_t *counts16) {
  memset(counts16, 0, 16 * sizeof(uint64_t));
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < k; ++j) counts16[(q[i * ld + j] >> 3) & 0xF]++;
}

int64_t nwc_oracle_fp8_encode(const uint8_t *q, int64_t n, int64_t k, int64_t ld, const uint8_t *sym_to_rank,
                              uint64_t *stream, int64_t stream_words, int64_t *row_start) {
  memset(stream, 0, (size_t)stream_words * sizeof(uint64_t));
  const int64_t cap = stream_words * 64;
  int64_t p = 0;
  for (int64_t i = 0; i < n; ++i) {
    row_start[i] = p;
    for (int64_t j = 0; j < k; ++j) {
      const unsigned b = q[i * ld + j];
      const unsigned sign = b >> 7, E = (b >> 3) & 0xF, M = b & 7, r = sym_to_rank[E];
      if (p + 16 > cap) return -1;
      if (r < ESCAPE_RANKS) {
        for (unsigned t = 0; t < r; ++t) put_bit(stream, p++, 1);
        put_bit(stream, p++, 0);
        put_bit(stream, p++, sign);
      } else {
        for (unsigned t = 0; t < ESCAPE_RANKS; ++t) put_bit(stream, p++, 1);
        put_bit(stream, p++, sign);
        for (unsigned t = 0; t < 4; ++t) put_bit(stream, p++, (E >> t) & 1u);
      }
      for (unsigned t = 0; t < 3; ++t) put_bit(stream, p++, (M >> t) & 1u);
    }
  }
  row_start[n] = p;
  return p;
}

int nwc_oracle_fp8_decode(const uint64_t *stream, const int64_t *row_start, int64_t n, int64_t k,
                          const uint8_t *rank_to_sym, uint8_t *out, int64_t ldo) {
  for (int64_t i = 0; i < n; ++i) {
    int64_t p = row_start[i];
    const int64_t end = row_start[i + 1];
    for (int64_t j = 0; j < k; ++j) {
      unsigned ones = 0;
      while (ones < ESCAPE_RANKS && p < end && get_bit(stream, p)) {
        ++ones;
        ++p;
      }
      unsigned sign, E, M = 0;
      if (ones < ESCAPE_RANKS) {
        if (p + 5 > end) return -1;
        ++p; /* the terminating zero */
        sign = get_bit(stream, p++);
        E = rank_to_sym[ones];
      } else {
        if (p + 8 > end) return -1;
        sign = get_bit(stream, p++);
        E = 0;
        for (unsigned t = 0; t < 4; ++t) E |= get_bit(stream, p++) << t;
      }
      for (unsigned t = 0; t < 3; ++t) M |= get_bit(stream, p++) << t;
      out[i * ldo + j] = (uint8_t)((sign << 7) | (E << 3) | M);
    }
    if (p != end) return -1;
  }
  return 0;
}

/* e4m3fn value: bias 7, subnormals M * 2^-9, S.1111.111 is NaN, no infinities. */
static double e4m3fn_value(uint8_t b) {
  const unsigned s = b >> 7, E = (b >> 3) & 0xF, M = b & 7;
  if (E == 15 && M == 7) return NAN;
  const double mag = E == 0 ? ldexp((double)M, -9) : ldexp(1.0 + M / 8.0, (int)E - 7);
  return s ? -mag : mag;
}

/* Model card: y_i = s_i * sum_j q_ij x_j, the per-channel scale applied after
 * the row sum; a_i = |s_i| * sum_j |q_ij x_j|. */
void nwc_oracle_fp8_matvec(const uint8_t *q, int64_t n, int64_t k, int64_t ld, const float *scale, const uint16_t *x,
                           double *y, double *a) {
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0, t = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      const double p = e4m3fn_value(q[i * ld + j]) * bf16_value(x[j]);
      s += p;
      t += fabs(p);
    }
    y[i] = (double)scale[i] * s;
    a[i] = fabs((double)scale[i]) * t;
  }
}
