"""Plain reference implementation of the NWC-style code and the batch-1 matvec.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and obvious on
purpose: scalar pure-Python versions for tiny inputs, and numpy versions that
are vectorised across rows only (never blocked, tiled or fused) for the larger
workloads.  Each function cites the passage of the pages it follows.

Stream organisation of this oracle: one bit stream per matrix row, codes in
column order, bits appended least-significant-first.  This is the oracle's
own layout; the library lays its streams out differently (the code, not the
layout, is the method).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "R_BF16", "R_FP8", "split_bf16", "join_bf16", "rank_table", "codeword_bf16",
    "code_length_bf16", "encode_bf16_scalar", "decode_bf16_scalar", "encode_bf16",
    "decode_bf16", "decode_bf16_rows", "coded_bits_closed_form_bf16", "byte_entropy",
    "kraft_sum_bf16", "parse_one_bf16", "bf16_value", "matvec_bf16_ref",
    "split_fp8", "codeword_fp8", "code_length_fp8", "encode_fp8", "decode_fp8",
    "fp8_e4m3fn_value", "matvec_fp8_ref", "gather_bf16_ref", "coded_bits_closed_form_fp8",
    "HUFF_MAX_LEN", "huffman_lengths_limited", "canonical_codes", "kraft_sum", "codeword_huffman",
    "encode_fp8_huffman", "decode_fp8_huffman",
]

# Escape threshold.  The pages say only "escape for rare values" (PyPI page,
# "How it works", second bullet).  Reading taken: the eight most frequent
# symbols get unary codes of length 1..8 (plus the sign), every other symbol
# is the escape prefix of eight ones followed by the sign and the raw symbol.
# For BF16 that makes the escape exactly 16 bits.
R_BF16 = 8
R_FP8 = 8


# ---------------------------------------------------------------------------
# Byte planes (PyPI page, "How it works", first bullet: a BF16 weight is its
# "mantissa byte", stored raw, and its "exponent/sign byte", entropy-coded).
# Reading taken: the BF16 high byte (sign + upper 7 exponent bits) is the
# exponent/sign byte; the low byte (exponent LSB + 7 mantissa bits) is the
# mantissa byte.  This split reproduces the page's entropy figures (about
# 7.97 bits for the raw byte, 2.6-2.9 bits for the coded one), which the
# tests check on the synthetic data.
# ---------------------------------------------------------------------------
def split_bf16(u):
    """(sign, 7-bit exponent symbol, mantissa byte) of BF16 bit patterns."""
    u = np.asarray(u, dtype=np.uint16)
    return (u >> 15) & 1, (u >> 8) & 0x7F, u & 0xFF


def join_bf16(s, e, m):
    s = np.asarray(s, np.uint16)
    e = np.asarray(e, np.uint16)
    m = np.asarray(m, np.uint16)
    return ((s << 15) | (e << 8) | m).astype(np.uint16)


# ---------------------------------------------------------------------------
# Frequency ranking (PyPI page, "How it works", second bullet: "ranked by
# frequency"; model card "How it was made": the coding is done per matrix).
# Tie-break (pages silent): equal counts are ordered by ascending symbol.
# Every symbol of the alphabet gets a rank, so any value can be coded.
# ---------------------------------------------------------------------------
def rank_table(counts):
    """(rank_to_sym, sym_to_rank) for a histogram over the alphabet."""
    counts = [int(c) for c in counts]
    order = sorted(range(len(counts)), key=lambda sym: (-counts[sym], sym))
    rank_to_sym = np.array(order, dtype=np.int64)
    sym_to_rank = np.empty(len(counts), dtype=np.int64)
    sym_to_rank[rank_to_sym] = np.arange(len(counts))
    return rank_to_sym, sym_to_rank


# ---------------------------------------------------------------------------
# Codeword (PyPI page, "How it works", second bullet: unary rank code plus a
# raw sign bit, escape for rare values).  Readings taken (pages silent on bit
# level): rank r < R is r one-bits then a zero-bit, then the sign; rank >= R is
# R one-bits, the sign, then the 7 symbol bits least-significant first.  The
# rank-0 code with its sign is 2 bits, which is what a padding filler costs on
# the same page ("Fused kernel" bullet).
# ---------------------------------------------------------------------------
def codeword_bf16(rank: int, s: int, e: int, R: int = R_BF16) -> list:
    """Bits of one codeword in stream order."""
    if rank < R:
        return [1] * rank + [0, int(s)]
    return [1] * R + [int(s)] + [(int(e) >> i) & 1 for i in range(7)]


def code_length_bf16(rank: int, R: int = R_BF16) -> int:
    return rank + 2 if rank < R else R + 8


def kraft_sum_bf16(R: int = R_BF16) -> float:
    """Kraft sum of the symbol part (sign excluded) over all 128 symbols."""
    from fractions import Fraction
    tot = Fraction(0)
    for r in range(128):
        tot += Fraction(1, 2 ** (code_length_bf16(r, R) - 1))
    return tot


def parse_one_bf16(bits, pos: int, rank_to_sym, R: int = R_BF16):
    """Decode one codeword starting at ``pos``: returns (s, e, new_pos)."""
    r = 0
    while r < R and bits[pos + r] == 1:
        r += 1
    if r < R:
        s = bits[pos + r + 1]
        return int(s), int(rank_to_sym[r]), pos + r + 2
    s = bits[pos + R]
    e = 0
    for i in range(7):
        e |= int(bits[pos + R + 1 + i]) << i
    return int(s), e, pos + R + 8


# ---------------------------------------------------------------------------
# Scalar codec: pure Python, tiny shapes only.
# ---------------------------------------------------------------------------
def encode_bf16_scalar(w_u16, R: int = R_BF16) -> dict:
    w = np.asarray(w_u16, dtype=np.uint16)
    n, k = w.shape
    s, e, m = split_bf16(w)
    counts = np.bincount(e.reshape(-1).astype(np.int64), minlength=128)
    r2s, s2r = rank_table(counts)
    rows = []
    for i in range(n):
        bits = []
        for j in range(k):
            bits += codeword_bf16(int(s2r[e[i, j]]), int(s[i, j]), int(e[i, j]), R)
        rows.append(bits)
    return dict(kind="bf16", n=n, k=k, R=R, counts=counts, rank_to_sym=r2s,
                sym_to_rank=s2r, rows=rows, mant=m.astype(np.uint8))


def decode_bf16_scalar(enc: dict) -> np.ndarray:
    n, k, R = enc["n"], enc["k"], enc["R"]
    out = np.empty((n, k), dtype=np.uint16)
    for i in range(n):
        bits = list(enc["rows"][i]) + [0] * 32
        pos = 0
        for j in range(k):
            s, e, pos = parse_one_bf16(bits, pos, enc["rank_to_sym"], R)
            out[i, j] = (s << 15) | (e << 8) | int(enc["mant"][i, j])
        assert pos == len(enc["rows"][i])
    return out


# ---------------------------------------------------------------------------
# numpy codec: per-row streams in one flat bit array (one uint8 per bit),
# vectorised across rows.
# ---------------------------------------------------------------------------
def _code_tables_bf16(s2r, R):
    val = np.zeros(256, dtype=np.uint32)
    ln = np.zeros(256, dtype=np.int64)
    for h in range(256):
        bits = codeword_bf16(int(s2r[h & 0x7F]), h >> 7, h & 0x7F, R)
        val[h] = sum(b << i for i, b in enumerate(bits))
        ln[h] = len(bits)
    return val, ln


def _pack_rows(hi_idx, val, ln, n, k):
    L = ln[hi_idx]
    V = val[hi_idx]
    row_bits = L.sum(axis=1)
    row_off = np.zeros(n, dtype=np.int64)
    if n > 1:
        row_off[1:] = np.cumsum(row_bits)[:-1]
    pos = row_off[:, None] + (np.cumsum(L, axis=1) - L)
    total = int(row_bits.sum())
    bits = np.zeros(total + 64, dtype=np.uint8)
    for b in range(int(ln.max())):
        sel = L > b
        bits[pos[sel] + b] = ((V[sel] >> b) & 1).astype(np.uint8)
    return bits, row_off, row_bits


def encode_bf16(w_u16, R: int = R_BF16) -> dict:
    """Encode a BF16 matrix: rank table, per-row code streams, mantissa plane."""
    w = np.ascontiguousarray(w_u16, dtype=np.uint16)
    n, k = w.shape
    hi = (w >> 8).astype(np.int64)
    counts = np.bincount((hi & 0x7F).reshape(-1), minlength=128)
    r2s, s2r = rank_table(counts)
    val, ln = _code_tables_bf16(s2r, R)
    bits, row_off, row_bits = _pack_rows(hi, val, ln, n, k)
    return dict(kind="bf16", n=n, k=k, R=R, counts=counts, rank_to_sym=r2s,
                sym_to_rank=s2r, bits=bits, row_off=row_off, row_bits=row_bits,
                mant=(w & 0xFF).astype(np.uint8),
                coded_bits=int(row_bits.sum()) + 8 * n * k)


def decode_bf16_rows(enc: dict, rows) -> np.ndarray:
    """Decode the listed rows (vectorised across them); returns uint16 [len(rows), K]."""
    rows = np.asarray(rows, dtype=np.int64)
    R, k = enc["R"], enc["k"]
    bits, r2s = enc["bits"], enc["rank_to_sym"]
    pos = enc["row_off"][rows].copy()
    mant = enc["mant"][rows].astype(np.uint16)
    out = np.empty((len(rows), k), dtype=np.uint16)
    for j in range(k):
        ones = np.zeros(len(rows), dtype=np.int64)
        run = np.ones(len(rows), dtype=bool)
        for t in range(R):
            run &= bits[pos + t] == 1
            ones += run
        esc = ones == R
        s = np.where(esc, bits[pos + R], bits[pos + np.minimum(ones, R - 1) + 1]).astype(np.uint16)
        pay = np.zeros(len(rows), dtype=np.int64)
        if esc.any():
            for i in range(7):
                pay |= bits[pos + R + 1 + i].astype(np.int64) << i
        e = np.where(esc, pay, r2s[np.minimum(ones, R - 1)]).astype(np.uint16)
        pos += np.where(esc, R + 8, ones + 2)
        out[:, j] = (s << 15) | (e << 8) | mant[:, j]
    assert np.array_equal(pos, enc["row_off"][rows] + enc["row_bits"][rows])
    return out


def decode_bf16(enc: dict) -> np.ndarray:
    return decode_bf16_rows(enc, np.arange(enc["n"]))


def coded_bits_closed_form_bf16(counts, sym_to_rank, n_weights: int, R: int = R_BF16) -> int:
    """Sum over symbols of count x code length, plus 8 raw bits per weight."""
    return int(sum(int(c) * code_length_bf16(int(sym_to_rank[e]), R)
                   for e, c in enumerate(counts))) + 8 * int(n_weights)


def byte_entropy(values, alphabet: int = 256) -> float:
    """Empirical Shannon entropy in bits of a byte-valued array."""
    c = np.bincount(np.asarray(values, dtype=np.int64).reshape(-1), minlength=alphabet)
    p = c[c > 0] / c.sum()
    return float(-(p * np.log2(p)).sum())


# ---------------------------------------------------------------------------
# Matvec (PyPI page, "Fused kernel" bullet: row sums of weight x activation
# for batch 1).  Plain definition, accumulated in float64:
#   y_i = sum_j w_ij x_j,   A_i = sum_j |w_ij x_j|   (A bounds the rounding).
# ---------------------------------------------------------------------------
def bf16_value(u16) -> np.ndarray:
    """Exact value of BF16 patterns as float64 (the pattern is the top half of an fp32)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def matvec_bf16_ref(w_u16, x_u16):
    """(y, A) in float64 for a BF16 matrix (bit patterns) and BF16 activation."""
    w = bf16_value(w_u16)
    x = bf16_value(x_u16)
    return w @ x, np.abs(w) @ np.abs(x)


def gather_bf16_ref(enc: dict, ids) -> np.ndarray:
    """Rows ``ids`` of the encoded matrix, decoded; ids outside [0, N) give zero rows."""
    ids = np.asarray(ids, dtype=np.int64)
    ok = (ids >= 0) & (ids < enc["n"])
    out = np.zeros((len(ids), enc["k"]), dtype=np.uint16)
    if ok.any():
        uniq, inv = np.unique(ids[ok], return_inverse=True)
        out[ok] = decode_bf16_rows(enc, uniq)[inv]
    return out


# ---------------------------------------------------------------------------
# fp8 e4m3fn variant (model card "Qwen3-4B-NWC-fp8": weight-only fp8 with a
# symmetric per-output-channel scale; the fp8 values are entropy-coded and
# come back bit for bit; the scale is applied at the end of the row sum).
# Reading taken: the 4-bit exponent field is the ranked symbol; sign and the 3
# mantissa bits follow the unary code raw, inside the same stream, so the
# whole byte is coded.  Escape: R ones, sign, 4 exponent bits, 3 mantissa bits.
# ---------------------------------------------------------------------------
def split_fp8(b):
    b = np.asarray(b, dtype=np.uint8)
    return (b >> 7) & 1, (b >> 3) & 0xF, b & 7


def codeword_fp8(rank: int, s: int, E: int, M: int, R: int = R_FP8) -> list:
    mbits = [(int(M) >> i) & 1 for i in range(3)]
    if rank < R:
        return [1] * rank + [0, int(s)] + mbits
    return [1] * R + [int(s)] + [(int(E) >> i) & 1 for i in range(4)] + mbits


def code_length_fp8(rank: int, R: int = R_FP8) -> int:
    return rank + 5 if rank < R else R + 8


def encode_fp8(q_u8, R: int = R_FP8) -> dict:
    q = np.ascontiguousarray(q_u8, dtype=np.uint8)
    n, k = q.shape
    E = ((q >> 3) & 0xF).astype(np.int64)
    counts = np.bincount(E.reshape(-1), minlength=16)
    r2s, s2r = rank_table(counts)
    val = np.zeros(256, dtype=np.uint32)
    ln = np.zeros(256, dtype=np.int64)
    for b in range(256):
        bits = codeword_fp8(int(s2r[(b >> 3) & 0xF]), b >> 7, (b >> 3) & 0xF, b & 7, R)
        val[b] = sum(v << i for i, v in enumerate(bits))
        ln[b] = len(bits)
    bits, row_off, row_bits = _pack_rows(q.astype(np.int64), val, ln, n, k)
    return dict(kind="fp8", n=n, k=k, R=R, counts=counts, rank_to_sym=r2s,
                sym_to_rank=s2r, bits=bits, row_off=row_off, row_bits=row_bits,
                coded_bits=int(row_bits.sum()))


def decode_fp8(enc: dict) -> np.ndarray:
    n, k, R = enc["n"], enc["k"], enc["R"]
    bits, r2s = enc["bits"], enc["rank_to_sym"]
    pos = enc["row_off"].copy()
    out = np.empty((n, k), dtype=np.uint8)
    for j in range(k):
        ones = np.zeros(n, dtype=np.int64)
        run = np.ones(n, dtype=bool)
        for t in range(R):
            run &= bits[pos + t] == 1
            ones += run
        esc = ones == R
        base = np.where(esc, pos + R, pos + ones + 1)       # position of the sign bit
        s = bits[base].astype(np.int64)
        Epay = np.zeros(n, dtype=np.int64)
        for i in range(4):
            Epay |= bits[base + 1 + i].astype(np.int64) << i
        mpos = np.where(esc, base + 5, base + 1)
        M = np.zeros(n, dtype=np.int64)
        for i in range(3):
            M |= bits[mpos + i].astype(np.int64) << i
        E = np.where(esc, Epay, r2s[np.minimum(ones, R - 1)])
        pos = mpos + 3
        out[:, j] = ((s << 7) | (E << 3) | M).astype(np.uint8)
    assert np.array_equal(pos, enc["row_off"] + enc["row_bits"])
    return out


def coded_bits_closed_form_fp8(counts, sym_to_rank, R: int = R_FP8) -> int:
    return int(sum(int(c) * code_length_fp8(int(sym_to_rank[E]), R) for E, c in enumerate(counts)))


def fp8_e4m3fn_value(b) -> np.ndarray:
    """float64 value of e4m3fn bytes: bias 7, subnormals M*2^-9, S.1111.111 is NaN, no infinities."""
    s, E, M = split_fp8(b)
    s = s.astype(np.float64)
    E = E.astype(np.int64)
    M = M.astype(np.float64)
    mag = np.where(E == 0, M * 2.0 ** -9, (1.0 + M / 8.0) * np.exp2((E - 7).astype(np.float64)))
    v = np.where(s == 1, -mag, mag)
    return np.where((E == 15) & (M == 7), np.nan, v)


def matvec_fp8_ref(q_u8, scale_f32, x_u16):
    """(y, A): y_i = s_i * sum_j q_ij x_j in float64; A_i = |s_i| * sum_j |q_ij x_j|."""
    q = fp8_e4m3fn_value(q_u8)
    x = bf16_value(x_u16)
    s = np.asarray(scale_f32, dtype=np.float32).astype(np.float64)
    return s * (q @ x), np.abs(s) * (np.abs(q) @ np.abs(x))


# ---------------------------------------------------------------------------
# fp8 coder variant: a length-limited canonical Huffman code over whole fp8
# bytes.  The model card "Qwen3-4B-NWC-fp8" (summary) codes the fp8 bytes
# whole; the third-party article (section on the limits of lossless weight
# compression) puts the current coder's saving well below the ideal.  Readings
# taken: every byte that occurs gets an optimal prefix code with no codeword
# longer than max_len bits (found by package-merge); canonical codewords
# (symbols in order of (length, byte); first all zeros; each next = previous
# + 1, shifted left by the growth in length); codewords written most
# significant bit first.  max_len = 12 is the library's decode-table peek.
# ---------------------------------------------------------------------------
HUFF_MAX_LEN = 12


def huffman_lengths_limited(counts, max_len: int = HUFF_MAX_LEN) -> list:
    """Optimal code lengths (at most max_len bits) of the symbols with a nonzero count, by package-merge.

    Leaves are the symbols, weighted by count.  Starting from the sorted
    leaves, max_len - 1 times: pair neighbours into packages (weight sum) and
    merge the packages with the leaves in weight order.  The first 2n - 2 items
    of the final list are the chosen ones; a symbol's length is the number of
    chosen items it appears in.  A lone symbol gets length 1."""
    counts = [int(c) for c in counts]
    syms = [s for s in range(len(counts)) if counts[s] > 0]
    lengths = [0] * len(counts)
    if not syms:
        return lengths
    if len(syms) == 1:
        lengths[syms[0]] = 1
        return lengths
    if (1 << max_len) < len(syms):
        raise ValueError("too many symbols for the length limit")
    leaves = sorted(((counts[s], (s,)) for s in syms), key=lambda t: (t[0], t[1]))
    cur = list(leaves)
    for _ in range(max_len - 1):
        packages = [(cur[i][0] + cur[i + 1][0], cur[i][1] + cur[i + 1][1]) for i in range(0, len(cur) - 1, 2)]
        cur = sorted(leaves + packages, key=lambda t: t[0])  # stable: leaves before equal packages
    for _, members in cur[:2 * len(syms) - 2]:
        for s in members:
            lengths[s] += 1
    return lengths


def canonical_codes(lengths) -> dict:
    """{symbol: (codeword value, length)} of the canonical code with these lengths (0 = no codeword)."""
    order = sorted((l, s) for s, l in enumerate(lengths) if l > 0)
    codes, code, prev = {}, 0, None
    for l, s in order:
        if prev is not None:
            code = (code + 1) << (l - prev)
        codes[s] = (code, l)
        prev = l
    return codes


def kraft_sum(lengths):
    from fractions import Fraction
    return sum(Fraction(1, 2 ** l) for l in lengths if l > 0)


def codeword_huffman(code: int, length: int) -> list:
    """Bits of a codeword in stream order (most significant bit first)."""
    return [(code >> (length - 1 - i)) & 1 for i in range(length)]


def encode_fp8_huffman(q_u8, max_len: int = HUFF_MAX_LEN, filler_codeword: bool = True) -> dict:
    """Per-row streams of the fp8 bytes under the matrix's length-limited canonical Huffman code.

    filler_codeword: give byte 0x00 a codeword even when it does not occur
    (counted once) -- the library pads its lane streams with that byte; the
    oracle's own streams need no padding, so a worked example may turn it off."""
    q = np.ascontiguousarray(q_u8, dtype=np.uint8)
    n, k = q.shape
    counts = np.bincount(q.reshape(-1).astype(np.int64), minlength=256)
    cons = counts.copy()
    if filler_codeword and cons[0] == 0:
        cons[0] = 1
    lengths = huffman_lengths_limited(cons, max_len)
    codes = canonical_codes(lengths)
    val = np.zeros(256, dtype=np.uint32)
    ln = np.zeros(256, dtype=np.int64)
    for s, (c, l) in codes.items():
        bits = codeword_huffman(c, l)
        val[s] = sum(b << i for i, b in enumerate(bits))
        ln[s] = l
    bits, row_off, row_bits = _pack_rows(q.astype(np.int64), val, ln, n, k)
    return dict(kind="fp8_huffman", n=n, k=k, counts=counts, lengths=np.array(lengths), max_len=max_len,
                bits=bits, row_off=row_off, row_bits=row_bits, coded_bits=int(row_bits.sum()))


def decode_fp8_huffman(enc: dict) -> np.ndarray:
    """Canonical decode, vectorised across rows: read bits one by one, MSB first, until the value read is a
    codeword of the current length (codewords of length l are the values first[l] .. first[l] + count[l] - 1)."""
    n, k, L = enc["n"], enc["k"], enc["max_len"]
    lengths = [int(v) for v in enc["lengths"]]
    codes = canonical_codes(lengths)
    first = np.zeros(L + 2, dtype=np.int64)
    num = np.zeros(L + 2, dtype=np.int64)
    sym_at = {}
    for s, (c, l) in codes.items():
        num[l] += 1
        sym_at[(l, c)] = s
    for l in range(1, L + 1):
        cs = [c for (ll, c) in sym_at if ll == l]
        first[l] = min(cs) if cs else 0
    table = np.full((L + 1, 1 << L), -1, dtype=np.int64)
    for (l, c), s in sym_at.items():
        table[l, c] = s
    bits = enc["bits"]
    pos = enc["row_off"].copy()
    out = np.empty((n, k), dtype=np.uint8)
    for j in range(k):
        code = np.zeros(n, dtype=np.int64)
        sym = np.full(n, -1, dtype=np.int64)
        used = np.zeros(n, dtype=np.int64)
        for l in range(1, L + 1):
            live = sym < 0
            code = np.where(live, (code << 1) | bits[pos + l - 1], code)
            hit = live & (table[l, np.minimum(code, (1 << L) - 1)] >= 0) & (code < (1 << l))
            sym = np.where(hit, table[l, np.minimum(code, (1 << L) - 1)], sym)
            used = np.where(hit, l, used)
        assert (sym >= 0).all(), "stream does not parse"
        pos += used
        out[:, j] = sym.astype(np.uint8)
    assert np.array_equal(pos, enc["row_off"] + enc["row_bits"])
    return out
