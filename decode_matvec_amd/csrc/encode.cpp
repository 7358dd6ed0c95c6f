// Host encoder and the host-only entry points of the C ABI.
//
// Follows the "neural-weight-compression 0.9.0" PyPI page, "How it works":
// byte planes (raw mantissa byte, coded exponent/sign byte), per-matrix
// frequency ranking, unary rank code with a raw sign bit and an escape; and
// the "Qwen3-4B-NWC-fp8" model card for fp8 bytes coded whole.  The stream
// layout (work items of R rows x 64/R column slices, one lane per slice) is
// described in nwc_format.h.
#include <algorithm>
#include <climits>
#include <utility>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "nwc_check.h"

namespace {

struct CodeTable {
  uint32_t val[256];  // codeword bits, first stream bit in bit 0
  uint8_t len[256];
};

int worker_count() {
  if (const char *s = std::getenv("NWC_ENCODE_THREADS")) {
    int v = std::atoi(s);
    if (v > 0) return std::min(v, 256);
  }
  unsigned hc = std::thread::hardware_concurrency();
  return (int)std::max(1u, std::min(hc, 64u));
}

// Runs f(begin, end) over [0, n) split across worker threads.
template <class F>
void parallel_for(int64_t n, F f) {
  const int t = (int)std::min<int64_t>(worker_count(), std::max<int64_t>(n, 1));
  if (t <= 1) {
    f((int64_t)0, n);
    return;
  }
  std::vector<std::thread> th;
  th.reserve(t);
  for (int i = 0; i < t; ++i) {
    const int64_t b = n * i / t, e = n * (i + 1) / t;
    th.emplace_back([=] { f(b, e); });
  }
  for (auto &x : th) x.join();
}

// Frequency rank: count descending, equal counts by ascending symbol.
void rank_table(const uint64_t *counts, int alphabet, uint8_t *rank_to_sym, uint8_t *sym_to_rank) {
  std::vector<int> order(alphabet);
  for (int i = 0; i < alphabet; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return counts[a] > counts[b]; });
  for (int r = 0; r < alphabet; ++r) {
    rank_to_sym[r] = (uint8_t)order[r];
    sym_to_rank[order[r]] = (uint8_t)r;
  }
}

// BF16 exponent/sign byte h = sign<<7 | symbol: rank r < 8 -> r ones, a zero,
// the sign; otherwise 8 ones, the sign, the 7 symbol bits.
void bf16_codes(const uint8_t *sym_to_rank, CodeTable &t) {
  for (int h = 0; h < 256; ++h) {
    const uint32_t s = h >> 7, e = h & 0x7F, r = sym_to_rank[e];
    if (r < NWC_ESCAPE_R) {
      t.val[h] = ((1u << r) - 1) | (s << (r + 1));
      t.len[h] = (uint8_t)(r + 2);
    } else {
      t.val[h] = 0xFFu | (s << 8) | (e << 9);
      t.len[h] = 16;
    }
  }
}

// fp8 byte b = sign<<7 | E<<3 | M: rank of E as unary, then sign and the 3
// mantissa bits; escape: 8 ones, sign, E (4 bits), M (3 bits).
void fp8_codes(const uint8_t *sym_to_rank, CodeTable &t) {
  for (int b = 0; b < 256; ++b) {
    const uint32_t s = b >> 7, E = (b >> 3) & 15, M = b & 7, r = sym_to_rank[E];
    if (r < NWC_ESCAPE_R) {
      t.val[b] = ((1u << r) - 1) | (s << (r + 1)) | (M << (r + 2));
      t.len[b] = (uint8_t)(r + 5);
    } else {
      t.val[b] = 0xFFu | (s << 8) | (E << 9) | (M << 13);
      t.len[b] = 16;
    }
  }
}

int trailing_ones(uint32_t v) { return v == 0xFFFFFFFFu ? 32 : __builtin_ctz(~v); }

// BF16 bit pattern of an e4m3fn byte (exact: every e4m3fn value is a BF16 value).
uint32_t fp8_to_bf16(uint32_t b) {
  const uint32_t s = (b >> 7) & 1, E = (b >> 3) & 15, M = b & 7;
  if (E == 15 && M == 7) return (s << 15) | 0x7FC0u;
  if (E == 0) {
    if (M == 0) return s << 15;
    int p = 31 - __builtin_clz(M);                     // M * 2^-9 = 2^(p-9) * (M / 2^p)
    return (s << 15) | ((uint32_t)(p + 118) << 7) | ((M ^ (1u << p)) << (7 - p));
  }
  return (s << 15) | ((E + 120) << 7) | (M << 4);
}

// Decode table for a 12-bit peek (layout in nwc_format.h).
void build_lut_bf16(const uint8_t *rank_to_sym, uint32_t *lut) {
  for (uint32_t p = 0; p < NWC_LUT_ENTRIES; ++p) {
    uint32_t entry = 0x80000000u;
    const int ra = trailing_ones(p);
    if (ra < NWC_ESCAPE_R) {
      const uint32_t la = ra + 2, sa = (p >> (ra + 1)) & 1;
      const uint32_t q = p >> la, avail = 12 - la;
      const int rb = trailing_ones(q);
      if (rb < NWC_ESCAPE_R && (uint32_t)rb + 2 <= avail) {
        const uint32_t lb = rb + 2, sb = (q >> (rb + 1)) & 1;
        const uint32_t ha = (sa << 7) | rank_to_sym[ra], hb = (sb << 7) | rank_to_sym[rb];
        entry = (la + lb) | (ha << 8) | (hb << 16);
      }
    }
    lut[p] = entry;
  }
}

void build_lut_fp8(const uint8_t *rank_to_sym, uint32_t *lut) {
  for (uint32_t p = 0; p < NWC_LUT_ENTRIES; ++p) {
    uint32_t entry = 0x80000000u;
    const int r = trailing_ones(p);
    if (r < NWC_ESCAPE_R) {  // r + 5 <= 12 bits: always complete
      const uint32_t s = (p >> (r + 1)) & 1, M = (p >> (r + 2)) & 7, E = rank_to_sym[r];
      const uint32_t b = (s << 7) | (E << 3) | M;
      entry = fp8_to_bf16(b) | (b << 16) | ((uint32_t)(r + 5) << 24);
    }
    lut[p] = entry;
  }
}

// ------------------------------------------------------------ Huffman variant
// Length-limited Huffman code over whole fp8 bytes (nwc_format.h, coder
// variant).  Lengths by package-merge: the present symbols, sorted by count,
// are the leaves; max_len - 1 times, neighbouring items are paired into
// packages and the packages merged back with the leaves in count order; of the
// final list the first 2n - 2 items are kept, and a symbol's length is the
// number of kept items that contain it.  Optimal among prefix codes with no
// codeword longer than max_len.  A lone symbol gets one bit.
void huffman_lengths(const uint64_t *counts, int alphabet, int max_len, uint8_t *len) {
  struct Item {
    uint64_t w;
    std::vector<uint16_t> syms;
  };
  std::vector<Item> leaves;
  for (int s = 0; s < alphabet; ++s) {
    len[s] = 0;
    if (counts[s]) leaves.push_back({counts[s], {(uint16_t)s}});
  }
  if (leaves.empty()) return;
  if (leaves.size() == 1) {
    len[leaves[0].syms[0]] = 1;
    return;
  }
  auto by_weight = [](const Item &a, const Item &b) { return a.w < b.w; };
  std::stable_sort(leaves.begin(), leaves.end(), by_weight);
  std::vector<Item> cur = leaves;
  for (int level = 1; level < max_len; ++level) {
    std::vector<Item> next = leaves;
    for (size_t i = 0; i + 1 < cur.size(); i += 2) {
      Item p{cur[i].w + cur[i + 1].w, cur[i].syms};
      p.syms.insert(p.syms.end(), cur[i + 1].syms.begin(), cur[i + 1].syms.end());
      next.push_back(std::move(p));
    }
    std::stable_sort(next.begin(), next.end(), by_weight);
    cur = std::move(next);
  }
  for (size_t i = 0; i < 2 * leaves.size() - 2; ++i)
    for (uint16_t s : cur[i].syms) len[s]++;
}

// Canonical codewords for the lengths: symbols in order of (length, value),
// the first all zeros, each next the previous plus one shifted left by the
// growth in length.  The table holds each codeword bit-reversed, so that the
// stream (least significant bit first) carries it most significant bit first.
void huffman_codes(const uint8_t *len, CodeTable &t) {
  std::vector<std::pair<int, int>> order;
  for (int b = 0; b < 256; ++b) {
    t.val[b] = 0;
    t.len[b] = len[b];
    if (len[b]) order.push_back({len[b], b});
  }
  std::sort(order.begin(), order.end());
  uint32_t code = 0;
  for (size_t i = 0; i < order.size(); ++i) {
    const int l = order[i].first, b = order[i].second;
    if (i) code = (code + 1) << (l - order[i - 1].first);
    uint32_t rev = 0;
    for (int j = 0; j < l; ++j) rev |= ((code >> j) & 1u) << (l - 1 - j);
    t.val[b] = rev;
  }
}

// Decode table of the Huffman variant: every peek whose first len[b] bits are
// byte b's codeword decodes to b (its BF16 value, the byte, the length).  Peeks
// that start no codeword (only when the code is incomplete, e.g. a single
// symbol) are flagged; a valid stream never meets one.
void build_lut_fp8_huffman(const uint8_t *len, uint32_t *lut) {
  CodeTable t;
  huffman_codes(len, t);
  for (uint32_t p = 0; p < NWC_LUT_ENTRIES; ++p) lut[p] = 0x80000000u;
  for (int b = 0; b < 256; ++b) {
    if (!len[b]) continue;
    for (uint32_t p = t.val[b]; p < NWC_LUT_ENTRIES; p += 1u << len[b])
      lut[p] = fp8_to_bf16((uint32_t)b) | ((uint32_t)b << 16) | ((uint32_t)len[b] << 24);
  }
}

void pack_nibbles(const uint8_t *len, uint8_t *out128) {
  for (int i = 0; i < 128; ++i) out128[i] = (uint8_t)((len[2 * i] & 15) | (len[2 * i + 1] << 4));
}
void unpack_nibbles(const uint8_t *in128, uint8_t *len) {
  for (int i = 0; i < 128; ++i) {
    len[2 * i] = in128[i] & 15;
    len[2 * i + 1] = in128[i] >> 4;
  }
}

// Work-item geometry of one matrix (see nwc_format.h).
struct Geo {
  int C = 0, R = 0, S = 0, W = 0, n_spans = 0;
  int64_t n_rg = 0, n_items = 0;
  int64_t lane_cols() const { return n_rg * R * (int64_t)n_spans * W * S * C; }
};

Geo make_geo(int64_t n, int64_t k, int C, int R, int max_waves) {
  Geo g;
  g.C = C;
  g.R = R;
  g.S = NWC_LANES / R;
  const int64_t waves_per_row = nwc_ceil_div(nwc_ceil_div(k, C), g.S);
  g.n_spans = (int)nwc_ceil_div(waves_per_row, max_waves);
  g.W = (int)nwc_ceil_div(waves_per_row, g.n_spans);
  g.n_rg = nwc_ceil_div(n, R);
  g.n_items = g.n_rg * g.n_spans * g.W;
  return g;
}

// Code rows a lane of C columns is likely to need, from the histogram: the
// mean stream length plus six standard deviations (fillers are short, so a
// full lane of real weights is the long case).  Only used to rule out
// geometries whose workgroup would not fit the decoder's LDS; the exact
// rows are planned afterwards.
struct RowEstimate {
  double mean = 0, var = 0;  // code bits per weight
  uint32_t rows(int C) const {
    const double bits = NWC_LEAD_BITS + C * mean + 6.0 * std::sqrt(C * var);
    return (uint32_t)std::ceil(bits / 32.0);
  }
};

// Automatic geometry.  Lanes decode C/2 (BF16) code pairs one after the
// other, so C bounds a wave's decode latency: C = 32, or 16 for matrices too
// small to give thousands of waves otherwise (wider C only when no 32-column
// geometry fits).  Among the row counts R whose row group fits one workgroup
// within the LDS budget, the cost is the stored lane columns (fillers count)
// times a penalty for workgroups far from 5 waves -- measured on MI355X
// across the Qwen-shaped matrices: 4-5 waves per workgroup were fastest,
// 8-10 took 5-20% longer, 2-3 (with padding) longer still.
// Relative cost of W waves per workgroup.  The matvec keeps at most 25 waves
// per compute unit, as floor(25 / W) workgroups of W waves, each with its own
// copy of the 16 KiB decode table.  Fitted to cold-cache timings on MI355X
// (Qwen-shaped matrices): time grows as (25 / waves)^0.45 when fewer waves
// fit, and by about 1.7 % per table copy a compute unit stages.
double wave_penalty(int W) {
  const int groups = std::max(1, 25 / W), waves = groups * W;
  return std::pow(25.0 / waves, 0.45) * (1.0 + 0.017 * groups);
}

Geo auto_geo(int64_t n, int64_t k, int C_req, int R_req, const RowEstimate &est) {
  std::vector<int> Cs, Rs;
  if (C_req) Cs = {C_req};
  else Cs = {16, 32, 48, 64};
  if (R_req) Rs = {R_req};
  else Rs = {64, 32, 16, 8, 4, 2, 1};
  // Measured on MI355X (Qwen-shaped matrices, cold cache): 16 columns per lane
  // is fastest (short items decode from a two-word register window and
  // pipeline better), 32 some 8 % slower; 48 and 64 only where nothing else fits.
  auto c_factor = [](int C) { return C == 16 ? 1.0 : C == 32 ? 1.08 : 1.25; };
  Geo best;
  double best_cost = 0;
  for (int C : Cs) {
    for (int R : Rs) {
      // 16 rows per wave is the matrix-core batch geometry: its workgroups
      // keep at most 12 waves, so that two of them share a compute unit under
      // the 25-wave cap (measured on MI355X, Qwen3-4B layer matrices at 8 /
      // 16 / 32 tokens: 91.3 / 103.3 / 144.8 us per layer with up to 16 waves,
      // 85.7 / 95.5 / 137.6 with up to 12, 98.1 / 105.5 / 136.8 with up to 8).
      const Geo g = make_geo(n, k, C, R, R == 16 ? 12 : NWC_MAX_WAVES);
      if (C_req && R_req) return g;
      if (g.n_spans != 1) continue;
      if (nwc_lds_bytes_for(g.W, g.R, est.rows(C)) > NWC_LDS_BUDGET) continue;
      const double cost = (double)g.lane_cols() * wave_penalty(g.W) * c_factor(C);
      if (!best.C || cost < best_cost) {  // ties keep the smaller C, then the larger R
        best = g;
        best_cost = cost;
      }
    }
  }
  if (best.C) return best;
  return make_geo(n, k, Cs.back(), R_req ? R_req : 1, NWC_MAX_WAVES);  // k > 65536: several spans
}

// Lane L of item `item`: matrix row and first column (may lie past n / k).
struct LaneSpan {
  int64_t row, c0;
};
inline LaneSpan lane_span(const Geo &g, int64_t item, int L) {
  const int64_t group = item / g.W, wave = item - group * g.W;
  const int64_t rg = group / g.n_spans, span = group - rg * g.n_spans;
  const int64_t q = (span * g.W + wave) * g.S + (L % g.S);
  return {rg * g.R + L / g.S, q * g.C};
}

inline uint32_t symbol_index(const void *w, int elem, int64_t idx) {
  return elem == NWC_BF16 ? (uint32_t)(((const uint16_t *)w)[idx] >> 8) : (uint32_t)((const uint8_t *)w)[idx];
}

// Bits of one lane's stream: lead bits, its real codes, filler codes.
uint64_t lane_bits(const void *w, int64_t n, int64_t k, int64_t ld, int elem, const CodeTable &tab, uint64_t filler,
                   const Geo &g, const LaneSpan &ls) {
  uint64_t bits = NWC_LEAD_BITS;
  const int64_t real = ls.row < n ? std::max<int64_t>(0, std::min<int64_t>(k - ls.c0, g.C)) : 0;
  const int64_t base = ls.row * ld + ls.c0;
  for (int64_t c = 0; c < real; ++c) bits += tab.len[symbol_index(w, elem, base + c)];
  return bits + filler * (uint64_t)(g.C - real);
}

// Longest lane stream (in 32-bit words) of every item.
std::vector<uint32_t> plan_rows(const void *w, int64_t n, int64_t k, int64_t ld, int elem, const CodeTable &tab,
                                uint64_t filler, const Geo &g) {
  std::vector<uint32_t> rows(g.n_items, 1);
  parallel_for(g.n_items, [&](int64_t i0, int64_t i1) {
    for (int64_t it = i0; it < i1; ++it) {
      uint64_t maxbits = NWC_LEAD_BITS;
      for (int L = 0; L < NWC_LANES; ++L)
        maxbits = std::max(maxbits, lane_bits(w, n, k, ld, elem, tab, filler, g, lane_span(g, it, L)));
      rows[it] = (uint32_t)nwc_ceil_div((int64_t)maxbits, 32);
    }
  });
  return rows;
}

int64_t lds_need(const Geo &g, uint32_t max_rows) { return nwc_lds_bytes_for(g.W, g.R, max_rows); }

int64_t bound_bytes(int64_t n, int64_t k, int elem, int C_req, int R_req) {
  // Worst case over every admissible geometry: 16 code bits per weight.
  int64_t worst = 0;
  for (int C = 16; C <= NWC_MAX_COLS; C += 16) {
    if (C_req && C != C_req) continue;
    for (int R = 1; R <= NWC_LANES; R *= 2) {
      if (R_req && R != R_req) continue;
      for (int mw = NWC_MAX_WAVES; mw >= 1; --mw) {
        const Geo g = make_geo(n, k, C, R, mw);
        const int64_t mant = elem == NWC_BF16 ? g.n_items * NWC_LANES * C : 0;
        const int64_t code = g.n_items * nwc_ceil_div(NWC_LEAD_BITS + 16 * (int64_t)C, 32) * 256;
        worst = std::max(worst, NWC_HEADER_BYTES + NWC_LUT_BYTES + nwc_round_up(g.n_items * 8, 256) + mant + code);
      }
    }
  }
  return worst;
}

bool valid_geometry_request(int C, int R) {
  if (C != 0 && (C < 16 || C > NWC_MAX_COLS || C % 16)) return false;
  if (R != 0 && (R < 1 || R > NWC_LANES || (R & (R - 1)))) return false;
  return true;
}

}  // namespace

extern "C" {

int nwc_version(void) { return NWC_VERSION; }

const char *nwc_status_string(int s) {
  switch (s) {
    case NWC_OK: return "ok";
    case NWC_ERR_ARG: return "invalid argument (null or misaligned pointer, bad enum)";
    case NWC_ERR_SHAPE: return "shape out of range";
    case NWC_ERR_CAPACITY: return "buffer or workspace too small";
    case NWC_ERR_FORMAT: return "not a valid blob of this format version";
    case NWC_ERR_HIP: return "HIP runtime error";
    case NWC_ERR_UNSUPPORTED: return "unsupported request";
    default: return "unknown status";
  }
}

int nwc_encode_bound(int64_t n, int64_t k, int elem, int cols_per_lane, int rows_per_wave, int64_t *max_bytes) {
  if (!max_bytes) return NWC_ERR_ARG;
  if (elem != NWC_BF16 && elem != NWC_FP8_E4M3) return NWC_ERR_ARG;
  if (!valid_geometry_request(cols_per_lane, rows_per_wave)) return NWC_ERR_ARG;
  if (n <= 0 || k <= 0 || n > ((int64_t)1 << 31) || k > ((int64_t)1 << 31)) return NWC_ERR_SHAPE;
  *max_bytes = bound_bytes(n, k, elem, cols_per_lane, rows_per_wave);
  return NWC_OK;
}

int nwc_encode(const void *w, int64_t n, int64_t k, int64_t ld, int elem, int cols_per_lane, int rows_per_wave,
               void *blob, int64_t blob_cap, int64_t *blob_size) {
  return nwc_encode_ex(w, n, k, ld, elem, NWC_CODER_UNARY, cols_per_lane, rows_per_wave, blob, blob_cap, blob_size);
}

int nwc_encode_ex(const void *w, int64_t n, int64_t k, int64_t ld, int elem, int coder, int cols_per_lane,
                  int rows_per_wave, void *blob, int64_t blob_cap, int64_t *blob_size) {
  if (!w || !blob || !blob_size) return NWC_ERR_ARG;
  if (elem != NWC_BF16 && elem != NWC_FP8_E4M3) return NWC_ERR_ARG;
  if (coder != NWC_CODER_UNARY && coder != NWC_CODER_HUFFMAN) return NWC_ERR_ARG;
  if (coder == NWC_CODER_HUFFMAN && elem != NWC_FP8_E4M3) return NWC_ERR_UNSUPPORTED;
  const bool huff = coder == NWC_CODER_HUFFMAN;
  if (!valid_geometry_request(cols_per_lane, rows_per_wave)) return NWC_ERR_ARG;
  if (n <= 0 || k <= 0 || ld < k || n > ((int64_t)1 << 31) || k > ((int64_t)1 << 31)) return NWC_ERR_SHAPE;

  // 1. histogram of the symbol each code carries, over the real weights:
  // the BF16 high byte, or the whole fp8 byte (the unary code ranks its 4-bit
  // exponent field, the Huffman variant the byte itself)
  std::vector<uint64_t> bytes(256, 0);
  {
    const int t = worker_count();
    std::vector<std::vector<uint64_t>> part(t, std::vector<uint64_t>(256, 0));
    std::vector<std::thread> th;
    for (int i = 0; i < t; ++i)
      th.emplace_back([&, i] {
        auto &h = part[i];
        for (int64_t r = n * i / t; r < n * (i + 1) / t; ++r) {
          if (elem == NWC_BF16) {
            const uint16_t *row = (const uint16_t *)w + r * ld;
            for (int64_t c = 0; c < k; ++c) h[row[c] >> 8]++;
          } else {
            const uint8_t *row = (const uint8_t *)w + r * ld;
            for (int64_t c = 0; c < k; ++c) h[row[c]]++;
          }
        }
      });
    for (auto &x : th) x.join();
    for (auto &h : part)
      for (int s = 0; s < 256; ++s) bytes[s] += h[s];
  }

  // 2. rank table (unary) or code lengths (Huffman), and codewords
  nwc_header_t hd;
  memset(&hd, 0, sizeof hd);
  CodeTable tab;
  uint64_t filler_bits;
  if (!huff) {
    const int alphabet = elem == NWC_BF16 ? 128 : 16;
    std::vector<uint64_t> counts(alphabet, 0);
    for (int b = 0; b < 256; ++b) counts[elem == NWC_BF16 ? (b & 0x7F) : ((b >> 3) & 15)] += bytes[b];
    uint8_t sym_to_rank[128] = {0};
    rank_table(counts.data(), alphabet, hd.rank_to_sym, sym_to_rank);
    if (elem == NWC_BF16)
      bf16_codes(sym_to_rank, tab);
    else
      fp8_codes(sym_to_rank, tab);
    filler_bits = elem == NWC_BF16 ? 2 : 5;  // rank 0, sign 0 (fp8: mantissa 0): all-zero bits
  } else {
    std::vector<uint64_t> cons(bytes);
    if (!cons[0]) cons[0] = 1;  // the filler byte always gets a codeword
    uint8_t len[256];
    huffman_lengths(cons.data(), 256, NWC_HUFF_MAX_LEN, len);
    pack_nibbles(len, hd.rank_to_sym);
    huffman_codes(len, tab);
    filler_bits = tab.len[0];
  }

  // 3. work-item geometry; fewer waves per workgroup (more column spans) if
  // the staged code rows of a workgroup would not fit the decoder's LDS.
  RowEstimate est;
  {
    double total = 0, s1 = 0, s2 = 0;
    for (int b = 0; b < 256; ++b) {
      const double l = tab.len[b];
      total += (double)bytes[b];
      s1 += (double)bytes[b] * l;
      s2 += (double)bytes[b] * l * l;
    }
    est.mean = s1 / total;
    est.var = std::max(0.0, s2 / total - est.mean * est.mean);
  }
  Geo g = auto_geo(n, k, cols_per_lane, rows_per_wave, est);
  std::vector<uint32_t> rows;
  for (int mw = NWC_MAX_WAVES;; --mw) {
    rows = plan_rows(w, n, k, ld, elem, tab, filler_bits, g);
    const uint32_t mx = *std::max_element(rows.begin(), rows.end());
    if (mx > NWC_ROWS_CAP) return NWC_ERR_UNSUPPORTED;  // cannot happen: C <= 64 needs <= 33 rows
    if (lds_need(g, mx) <= NWC_LDS_BUDGET) break;
    if (g.W == 1) return NWC_ERR_UNSUPPORTED;  // cannot happen: one wave needs < 26 KiB
    g = make_geo(n, k, g.C, g.R, std::min(mw - 1, g.W - 1));
  }

  // 4. layout
  hd.magic = NWC_MAGIC;
  hd.version = NWC_FORMAT_VERSION;
  hd.elem = (uint32_t)elem;
  hd.header_bytes = NWC_HEADER_BYTES;
  hd.n = n;
  hd.k = k;
  hd.cols_per_lane = (uint32_t)g.C;
  hd.rows_per_wave = (uint32_t)g.R;
  hd.waves_per_group = (uint32_t)g.W;
  hd.n_spans = (uint32_t)g.n_spans;
  hd.n_rowgroups = (uint32_t)g.n_rg;
  hd.n_items = (uint32_t)g.n_items;
  hd.max_rows = *std::max_element(rows.begin(), rows.end());
  hd.escape_r = huff ? 0u : NWC_ESCAPE_R;
  hd.off_lut = NWC_HEADER_BYTES;
  hd.off_items = hd.off_lut + NWC_LUT_BYTES;
  hd.off_mant = hd.off_items + (uint64_t)nwc_round_up(g.n_items * 8, 256);
  hd.mant_bytes = elem == NWC_BF16 ? (uint64_t)g.n_items * NWC_LANES * g.C : 0;
  hd.off_code = hd.off_mant + hd.mant_bytes;
  std::vector<uint32_t> code_off(g.n_items);
  uint64_t code_bytes = 0;
  for (int64_t i = 0; i < g.n_items; ++i) {
    code_off[i] = (uint32_t)code_bytes;
    code_bytes += (uint64_t)rows[i] * 256;
    if (code_bytes > 0xFFFFFFFFull) return NWC_ERR_SHAPE;  // item offsets are 32-bit
  }
  hd.code_bytes = code_bytes;
  hd.total_bytes = hd.off_code + code_bytes;
  if ((int64_t)hd.total_bytes > blob_cap) return NWC_ERR_CAPACITY;

  // 5. coded size of the real weights (sum of codeword lengths + raw bytes)
  uint64_t coded = 0;
  for (int b = 0; b < 256; ++b) coded += bytes[b] * tab.len[b];
  if (elem == NWC_BF16) coded += 8ull * (uint64_t)n * (uint64_t)k;
  hd.coded_bits = coded;

  // 6. write header, decode table, item table
  uint8_t *out = (uint8_t *)blob;
  memset(out, 0, hd.off_code);
  memcpy(out, &hd, sizeof hd);
  uint32_t *lut = (uint32_t *)(out + hd.off_lut);
  if (elem == NWC_BF16) {
    build_lut_bf16(hd.rank_to_sym, lut);
  } else if (huff) {
    uint8_t len[256];
    unpack_nibbles(hd.rank_to_sym, len);
    build_lut_fp8_huffman(len, lut);
  } else {
    build_lut_fp8(hd.rank_to_sym, lut);
  }
  uint32_t *items = (uint32_t *)(out + hd.off_items);
  for (int64_t i = 0; i < g.n_items; ++i) {
    items[2 * i] = code_off[i];
    items[2 * i + 1] = rows[i];
  }

  // 7. code and mantissa planes, one item per task (unary fillers are zero
  // bits, so they stay as cleared; Huffman fillers are byte 0x00's codeword)
  parallel_for(g.n_items, [&](int64_t i0, int64_t i1) {
    for (int64_t it = i0; it < i1; ++it) {
      uint32_t *code = (uint32_t *)(out + hd.off_code + code_off[it]);
      memset(code, 0, (size_t)rows[it] * 256);
      uint8_t *mant = nullptr;
      if (elem == NWC_BF16) {
        mant = out + hd.off_mant + (uint64_t)it * NWC_LANES * g.C;
        memset(mant, 0, (size_t)NWC_LANES * g.C);
      }
      for (int L = 0; L < NWC_LANES; ++L) {
        const LaneSpan ls = lane_span(g, it, L);
        const int64_t nc = (ls.row >= n || ls.c0 >= k) ? 0 : std::min<int64_t>(k - ls.c0, g.C);
        if (nc == 0 && !huff) continue;
        uint64_t acc = 0;
        uint32_t nbits = NWC_LEAD_BITS, word = 0;
        for (int64_t c = 0; c < (huff ? (int64_t)g.C : nc); ++c) {
          const int64_t idx = ls.row * ld + ls.c0 + c;
          const uint32_t sym = c < nc ? symbol_index(w, elem, idx) : 0u;  // Huffman filler: byte 0x00
          acc |= (uint64_t)tab.val[sym] << nbits;
          nbits += tab.len[sym];
          if (nbits >= 32) {
            code[(uint64_t)word * NWC_LANES + L] = (uint32_t)acc;
            acc >>= 32;
            nbits -= 32;
            ++word;
          }
          if (mant && c < nc) mant[((c >> 4) * NWC_LANES + L) * 16 + (c & 15)] = (uint8_t)((const uint16_t *)w)[idx];
        }
        if (nbits) code[(uint64_t)word * NWC_LANES + L] = (uint32_t)acc;
      }
    }
  });
  *blob_size = (int64_t)hd.total_bytes;
  return NWC_OK;
}

int nwc_blob_info(const void *blob, int64_t blob_bytes, nwc_info *info) {
  if (!blob || !info) return NWC_ERR_ARG;
  if (blob_bytes < NWC_HEADER_BYTES) return NWC_ERR_CAPACITY;
  nwc_header_t h;
  memcpy(&h, blob, sizeof h);
  const int st = nwc_check_header(&h);
  if (st != NWC_OK) return st;
  memset(info, 0, sizeof *info);
  info->n = h.n;
  info->k = h.k;
  info->elem = (int32_t)h.elem;
  info->cols_per_lane = (int32_t)h.cols_per_lane;
  info->rows_per_wave = (int32_t)h.rows_per_wave;
  info->waves_per_group = (int32_t)h.waves_per_group;
  info->n_spans = (int32_t)h.n_spans;
  info->n_items = (int32_t)h.n_items;
  info->max_rows = (int32_t)h.max_rows;
  info->coded_bits = h.coded_bits;
  info->total_bytes = h.total_bytes;
  info->code_bytes = h.code_bytes;
  info->mant_bytes = h.mant_bytes;
  info->table_bytes = h.off_mant;
  info->coder = h.escape_r == 0 ? NWC_CODER_HUFFMAN : NWC_CODER_UNARY;
  memcpy(info->rank_to_sym, h.rank_to_sym, 128);
  return NWC_OK;
}

int nwc_blob_check(const void *blob, int64_t blob_bytes) {
  if (!blob) return NWC_ERR_ARG;
  if (blob_bytes < NWC_HEADER_BYTES) return NWC_ERR_CAPACITY;
  nwc_header_t h;
  memcpy(&h, blob, sizeof h);
  const int st = nwc_check_header(&h);
  if (st != NWC_OK) return st;
  if ((uint64_t)blob_bytes < h.total_bytes) return NWC_ERR_CAPACITY;
  const uint8_t *b = (const uint8_t *)blob;
  std::vector<uint32_t> lut(NWC_LUT_ENTRIES);
  if (h.escape_r == 0) {
    // Huffman variant: lengths at most 12 bits, Kraft sum at most one (a
    // prefix code), a codeword for the filler byte 0x00.
    uint8_t len[256];
    unpack_nibbles(h.rank_to_sym, len);
    uint64_t kraft = 0;  // in units of 2^-12
    for (int b = 0; b < 256; ++b) {
      if (len[b] > NWC_HUFF_MAX_LEN) return NWC_ERR_FORMAT;
      if (len[b]) kraft += 1ull << (NWC_HUFF_MAX_LEN - len[b]);
    }
    if (!len[0] || kraft > (1ull << NWC_HUFF_MAX_LEN)) return NWC_ERR_FORMAT;
    build_lut_fp8_huffman(len, lut.data());
  } else {
    // The rank table orders every symbol once (128 exponent/sign symbols, or
    // the 16 fp8 exponent fields).
    const int n_sym = h.elem == NWC_BF16 ? 128 : 16;
    bool seen[128] = {};
    for (int r = 0; r < n_sym; ++r) {
      const int sym = h.rank_to_sym[r];
      if (sym >= n_sym || seen[sym]) return NWC_ERR_FORMAT;
      seen[sym] = true;
    }
    if (h.elem == NWC_BF16)
      build_lut_bf16(h.rank_to_sym, lut.data());
    else
      build_lut_fp8(h.rank_to_sym, lut.data());
  }
  // The decode table is the one the rank table (or the code lengths) defines.
  if (memcmp(lut.data(), b + h.off_lut, NWC_LUT_BYTES) != 0) return NWC_ERR_FORMAT;
  // Every item's code rows lie inside the code plane, whole 256-byte rows,
  // at least one and at most max_rows (the kernels size their buffers by it).
  for (uint64_t i = 0; i < h.n_items; ++i) {
    uint32_t e[2];
    memcpy(e, b + h.off_items + 8 * i, 8);
    const uint64_t off = e[0], rows = e[1];
    if (rows < 1 || rows > h.max_rows || off % 256 || off + rows * 256 > h.code_bytes) return NWC_ERR_FORMAT;
  }
  return NWC_OK;
}

int nwc_workspace_size(const void *header, int64_t *bytes) {
  if (!header || !bytes) return NWC_ERR_ARG;
  nwc_header_t h;
  memcpy(&h, header, sizeof h);
  const int st = nwc_check_header(&h);
  if (st != NWC_OK) return st;
  if (h.n_spans == 1) {
    *bytes = 0;
    return NWC_OK;
  }
  // fp32 partial sums [row][column span padded to a multiple of 4]
  *bytes = nwc_round_up((int64_t)h.n_rowgroups * h.rows_per_wave * nwc_round_up(h.n_spans, 4) * 4, 256);
  return NWC_OK;
}

}  // extern "C"
