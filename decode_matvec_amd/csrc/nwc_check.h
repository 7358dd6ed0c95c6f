// Host-side validation of a blob header (used by every entry point).
#pragma once
#include <stdint.h>
#include <string.h>

#include "nwc_format.h"
#include "../../include/nwc.h"

static inline int64_t nwc_ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static inline int64_t nwc_round_up(int64_t a, int64_t b) { return nwc_ceil_div(a, b) * b; }

// The format's bound on a workgroup's decoder LDS, used by the encoder to
// choose geometries and by the header check: two code regions per wave (with
// guard rows), two sets of cross-wave row sums and the static decode table.
// It is conservative: the kernels use one code region per wave plus their row
// sums, the decode table and, for fp8, the 1 KiB escape table.
static inline int64_t nwc_lds_bytes_for(int64_t waves, int64_t rows_per_wave, int64_t max_rows) {
  return 2 * (waves * (max_rows + NWC_GUARD_ROWS) * 256 + waves * rows_per_wave * 4) + NWC_LUT_BYTES;
}
static inline int64_t nwc_lds_bytes(const nwc_header_t *h) {
  return nwc_lds_bytes_for(h->waves_per_group, h->rows_per_wave, h->max_rows);
}

// Returns NWC_OK if `h` is a structurally valid header of this format version.
static inline int nwc_check_header(const nwc_header_t *h) {
  if (!h) return NWC_ERR_ARG;
  if (h->magic != NWC_MAGIC || h->version != NWC_FORMAT_VERSION || h->header_bytes != NWC_HEADER_BYTES)
    return NWC_ERR_FORMAT;
  if (h->elem != NWC_BF16 && h->elem != NWC_FP8_E4M3) return NWC_ERR_FORMAT;
  if (h->n <= 0 || h->k <= 0 || h->n > (int64_t)1 << 31 || h->k > (int64_t)1 << 31) return NWC_ERR_FORMAT;
  const int64_t C = h->cols_per_lane, R = h->rows_per_wave, W = h->waves_per_group, sp = h->n_spans;
  if (C < 16 || C > NWC_MAX_COLS || C % 16) return NWC_ERR_FORMAT;
  if (R < 1 || R > NWC_LANES || (R & (R - 1))) return NWC_ERR_FORMAT;
  if (W < 1 || W > NWC_MAX_WAVES || sp < 1) return NWC_ERR_FORMAT;
  const int64_t waves_per_row = nwc_ceil_div(nwc_ceil_div(h->k, C), NWC_LANES / R);
  if (sp * W < waves_per_row || sp * (W - 1) >= waves_per_row) return NWC_ERR_FORMAT;
  if (h->n_rowgroups != nwc_ceil_div(h->n, R)) return NWC_ERR_FORMAT;
  if ((int64_t)h->n_items != (int64_t)h->n_rowgroups * sp * W) return NWC_ERR_FORMAT;
  if (h->max_rows < 1 || h->max_rows > NWC_ROWS_CAP) return NWC_ERR_FORMAT;
  if (h->escape_r != NWC_ESCAPE_R && !(h->escape_r == 0 && h->elem == NWC_FP8_E4M3)) return NWC_ERR_FORMAT;
  if (nwc_lds_bytes(h) > NWC_LDS_BUDGET) return NWC_ERR_FORMAT;
  const uint64_t items_bytes = (uint64_t)nwc_round_up((int64_t)h->n_items * 8, 256);
  const uint64_t mant = h->elem == NWC_BF16 ? (uint64_t)h->n_items * NWC_LANES * C : 0;
  if (h->off_lut != NWC_HEADER_BYTES || h->off_items != h->off_lut + NWC_LUT_BYTES ||
      h->off_mant != h->off_items + items_bytes || h->mant_bytes != mant ||
      h->off_code != h->off_mant + h->mant_bytes || h->off_code % 256 ||
      h->total_bytes != h->off_code + h->code_bytes ||
      h->code_bytes > (uint64_t)h->n_items * h->max_rows * 256)
    return NWC_ERR_FORMAT;
  return NWC_OK;
}
