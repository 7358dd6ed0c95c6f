// Host-side validation of a blob header (used by every entry point).
#pragma once
#include <stdint.h>
#include <string.h>

#include "nwc_format.h"
#include "../../include/nwc.h"

static inline int64_t nwc_ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static inline int64_t nwc_round_up(int64_t a, int64_t b) { return nwc_ceil_div(a, b) * b; }

// Returns NWC_OK if `h` is a structurally valid header of this format version.
static inline int nwc_check_header(const nwc_header_t *h) {
  if (!h) return NWC_ERR_ARG;
  if (h->magic != NWC_MAGIC || h->version != NWC_FORMAT_VERSION || h->header_bytes != NWC_HEADER_BYTES)
    return NWC_ERR_FORMAT;
  if (h->elem != NWC_BF16 && h->elem != NWC_FP8_E4M3) return NWC_ERR_FORMAT;
  if (h->n <= 0 || h->k <= 0 || h->n > (int64_t)1 << 31 || h->k > (int64_t)1 << 31) return NWC_ERR_FORMAT;
  const int64_t C = h->cols_per_item;
  if (C < 16 || C > NWC_MAX_COLS || C % 16) return NWC_ERR_FORMAT;
  if (h->n_rowblocks != nwc_ceil_div(h->n, NWC_LANES)) return NWC_ERR_FORMAT;
  if (h->n_kspans != nwc_ceil_div(h->k, C)) return NWC_ERR_FORMAT;
  if ((int64_t)h->n_items != (int64_t)h->n_rowblocks * h->n_kspans) return NWC_ERR_FORMAT;
  if (h->last_cols != h->k - (int64_t)(h->n_kspans - 1) * C) return NWC_ERR_FORMAT;
  if (h->k_pad != (int64_t)(h->n_kspans - 1) * C + nwc_round_up(h->last_cols, 16)) return NWC_ERR_FORMAT;
  if (h->max_rows < 1 || h->max_rows > NWC_ROWS_CAP || h->escape_r != NWC_ESCAPE_R) return NWC_ERR_FORMAT;
  const uint64_t items_bytes = (uint64_t)nwc_round_up((int64_t)h->n_items * 8, 256);
  const uint64_t mant = h->elem == NWC_BF16 ? (uint64_t)h->n_rowblocks * NWC_LANES * h->k_pad : 0;
  if (h->off_lut != NWC_HEADER_BYTES || h->off_items != h->off_lut + NWC_LUT_BYTES ||
      h->off_mant != h->off_items + items_bytes || h->mant_bytes != mant ||
      h->off_code != h->off_mant + h->mant_bytes || h->off_code % 256 ||
      h->total_bytes != h->off_code + h->code_bytes ||
      h->code_bytes > (uint64_t)h->n_items * h->max_rows * 256)
    return NWC_ERR_FORMAT;
  return NWC_OK;
}
