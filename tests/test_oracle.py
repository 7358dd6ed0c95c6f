"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks the oracle against a fact fixed by the pages or by
mathematics: a hand-derived worked example, the Kraft inequality, the
rearrangement inequality by brute force, Shannon's bound and the pages' 2 %
gate, the pages' entropy figures, exact rational arithmetic, special cases
with closed-form answers, and library routines for the number formats.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth as S
from synth import configs as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_tiny_codes.txt")
GOLDEN_FP8 = os.path.join(os.path.dirname(__file__), "golden", "fp8_tiny_codes.txt")


def load_golden(path=GOLDEN, dtype=np.uint16):
    ex = {}
    lines = [l.strip() for l in open(path) if l.strip() and not l.startswith("#")]
    i = 0
    while i < len(lines):
        parts = lines[i].split()
        if parts[0] == "matrix":
            name, n, k = parts[1], int(parts[2]), int(parts[3])
            rows = [[int(v, 16) for v in lines[i + 1 + r].split()] for r in range(n)]
            ex.setdefault(name, {})["w"] = np.array(rows, dtype=dtype)
            i += 1 + n
            continue
        if parts[0] == "ranks":
            ex[parts[1]]["ranks"] = [int(v, 16) for v in parts[2:]]
        elif parts[0] == "rowbits":
            ex[parts[1]].setdefault("rowbits", {})[int(parts[2])] = [int(c) for c in parts[3]]
        elif parts[0] == "coded":
            ex[parts[1]]["coded"] = int(parts[2])
        i += 1
    return ex


# --------------------------------------------------------------- worked example
@pytest.mark.parametrize("name", ["A", "B"])
def test_golden_bitstreams(name):
    ex = load_golden()[name]
    enc_s = O.encode_bf16_scalar(ex["w"])
    enc_v = O.encode_bf16(ex["w"])
    assert list(enc_s["rank_to_sym"][:len(ex["ranks"])]) == ex["ranks"]
    for r, bits in ex["rowbits"].items():
        assert enc_s["rows"][r] == bits
        off, nb = enc_v["row_off"][r], enc_v["row_bits"][r]
        assert list(enc_v["bits"][off:off + nb]) == bits
    assert enc_v["coded_bits"] == ex["coded"]
    assert np.array_equal(O.decode_bf16_scalar(enc_s), ex["w"])
    assert np.array_equal(O.decode_bf16(enc_v), ex["w"])


# --------------------------------------------------------------- code structure
def test_kraft_and_prefix_free():
    # Symbol part (sign excluded): 8 unary codes 1..8 bits + 120 escapes of 15.
    k = O.kraft_sum_bf16()
    assert k == 1 - Fraction(1, 2 ** 8) + 120 * Fraction(1, 2 ** 15)
    assert k <= 1
    r2s = np.arange(128)
    words = {}
    for rank in range(128):
        for s in (0, 1):
            w = tuple(O.codeword_bf16(rank, s, int(r2s[rank])))
            assert len(w) == O.code_length_bf16(rank)
            words[w] = (rank, s)
    ws = list(words)
    for a in ws:
        for b in ws:
            if a is not b:
                assert a != b[:len(a)], "codeword is a prefix of another"


def test_every_short_string_parses_uniquely():
    # Brute force: every 16-bit string starts with exactly one codeword, and
    # parsing returns the codeword that generated it.
    r2s = np.arange(128)
    for v in range(1 << 16):
        bits = [(v >> i) & 1 for i in range(16)] + [0] * 8
        s, e, p = O.parse_one_bf16(bits, 0, r2s)
        rank = int(np.where(r2s == e)[0][0])
        if p - 0 < 16 or rank >= O.R_BF16:
            assert bits[:p] == O.codeword_bf16(rank, s, e)


def test_rank_order_minimises_length_bruteforce():
    rng = np.random.default_rng(7)
    for trial in range(30):
        a = int(rng.integers(2, 8))
        counts = rng.integers(0, 50, size=a)
        _, s2r = O.rank_table(counts)
        best = min(sum(int(counts[e]) * O.code_length_bf16(p[e]) for e in range(a))
                   for p in itertools.permutations(range(a)))
        got = sum(int(counts[e]) * O.code_length_bf16(int(s2r[e])) for e in range(a))
        assert got == best


# --------------------------------------------------------------- round trips
def _odd_mats():
    out = []
    for idx, (n, k) in enumerate(C.ODD_SHAPES):
        g = S.inject_rare(S.normal_bf16(C.odd_seed(2 * idx), (n, k), 0.02), C.odd_seed(2 * idx) + 50)
        t = S.inject_rare(S.student_t_bf16(C.odd_seed(2 * idx + 1), (n, k)), C.odd_seed(2 * idx + 1) + 50)
        out += [(f"normal_{n}x{k}", g), (f"t3_{n}x{k}", t)]
    out.append(("all_patterns", S.all_patterns_bf16()))
    return out


@pytest.mark.parametrize("name,w", _odd_mats(), ids=lambda v: v if isinstance(v, str) else "")
def test_roundtrip_odd_shapes(name, w):
    enc = O.encode_bf16(w)
    assert np.array_equal(O.decode_bf16(enc), w)
    assert enc["coded_bits"] == O.coded_bits_closed_form_bf16(enc["counts"], enc["sym_to_rank"], w.size)


def test_scalar_and_numpy_codecs_agree():
    w = S.inject_rare(S.normal_bf16(11, (9, 37), 0.02), 12, frac=0.05)
    a = O.encode_bf16_scalar(w)
    b = O.encode_bf16(w)
    for r in range(w.shape[0]):
        off, nb = b["row_off"][r], b["row_bits"][r]
        assert list(b["bits"][off:off + nb]) == a["rows"][r]
    assert np.array_equal(O.decode_bf16_scalar(a), w)


def test_all_patterns_ranks_are_symbols():
    # Every symbol occurs 512 times, so ties decide: rank == symbol value and
    # symbols >= 8 take the escape.
    enc = O.encode_bf16(S.all_patterns_bf16())
    assert list(enc["rank_to_sym"]) == list(range(128))
    assert enc["counts"].tolist() == [512] * 128


def test_single_matrix_roundtrip_and_size():
    w = S.normal_bf16(C.SINGLE["w_seed"], (1024, 1024), C.SINGLE["sigma"])
    enc = O.encode_bf16(w)
    rows = np.arange(0, 1024, 7)
    assert np.array_equal(O.decode_bf16_rows(enc, rows), w[rows])
    bits_from_hist = O.coded_bits_closed_form_bf16(enc["counts"], enc["sym_to_rank"], w.size)
    assert enc["coded_bits"] == bits_from_hist == int(enc["row_bits"].sum()) + 8 * w.size


def test_single_matrix_full_roundtrip():
    w = S.normal_bf16(C.SINGLE["w_seed"], (1024, 1024), C.SINGLE["sigma"])
    assert np.array_equal(O.decode_bf16(O.encode_bf16(w)), w)


# --------------------------------------------------------------- entropy figures
def _entropy_gate(w):
    s, e, m = O.split_bf16(w)
    h_hi = O.byte_entropy(w >> 8)
    h_lo = O.byte_entropy(m)
    enc = O.encode_bf16(w)
    ideal = w.size * (h_hi + 8.0)
    return h_hi, h_lo, enc["coded_bits"], ideal


@pytest.mark.parametrize("k", [2560, 4096, 9728])
def test_entropy_band_qwen_sigmas(k):
    # Shannon: no prefix code beats H(hi)+8 bits per weight.  Gate: within 2 %.
    w = S.normal_bf16(900 + k, (512, 2048), C.sigma_for(k))
    h_hi, h_lo, coded, ideal = _entropy_gate(w)
    assert ideal <= coded <= 1.02 * ideal
    # The pages' figures for BF16 LLM weights: 7.97 bits raw byte, 2.6-2.9 coded byte.
    assert abs(h_lo - 7.97) < 0.01
    assert 2.6 <= h_hi <= 2.9


@pytest.mark.parametrize("name,w", _odd_mats()[:-1], ids=lambda v: v if isinstance(v, str) else "")
def test_entropy_band_odd(name, w):
    h_hi, h_lo, coded, ideal = _entropy_gate(w)
    assert coded >= ideal
    if w.size >= 100000:
        assert coded <= 1.02 * ideal


def test_generator_exponent_histogram_chi2():
    # The 7-bit symbol e of a BF16 weight holds |w| in [2^(2e-127), 2^(2e-125))
    # (edges moved down by half an ulp by the round to nearest); compare the
    # empirical histogram of N(0, 0.02) draws with normal-CDF bin masses.
    from scipy.stats import norm, chi2
    sigma = 0.02
    w = S.normal_bf16(77, (1 << 20,), sigma)
    _, e, _ = O.split_bf16(w)
    cnt = np.bincount(e.astype(np.int64), minlength=128).astype(np.float64)
    lo = np.array([0.0] + [2.0 ** (2 * v - 127) * (1 - 2.0 ** -9) for v in range(1, 128)])
    hi = np.append(lo[1:], np.inf)
    p = 2 * (norm.cdf(hi / sigma) - norm.cdf(lo / sigma))
    n = cnt.sum()
    keep = p * n >= 20
    exp = np.append(p[keep] * n, p[~keep].sum() * n)
    obs = np.append(cnt[keep], cnt[~keep].sum())
    stat = ((obs - exp) ** 2 / np.maximum(exp, 1e-9)).sum()
    assert stat < chi2.ppf(0.999, df=len(obs) - 1)


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(5)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1e-3,
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, 3.4e38, 1.0 + 2 ** -8,
                                  1.0 + 3 * 2 ** -8], np.float32)])
    t = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(S.bf16_from_f32(a), t)


# --------------------------------------------------------------- matvec
def _exact(u16):
    v = O.bf16_value(u16)
    return [Fraction(float(t)) for t in v.reshape(-1)]


@pytest.mark.parametrize("n,k,seed", [(1, 1, 1), (3, 17, 2), (4, 600, 3), (2, 513, 4)])
def test_matvec_against_exact_rationals(n, k, seed):
    w = S.inject_rare(S.normal_bf16(seed, (n, k), 0.02), seed + 1, frac=0.01)
    x = S.activation_bf16(seed + 2, k)
    y, A = O.matvec_bf16_ref(w, x)
    W = _exact(w)
    X = _exact(x)
    for i in range(n):
        ye = sum(W[i * k + j] * X[j] for j in range(k))
        Ae = sum(abs(W[i * k + j] * X[j]) for j in range(k))
        assert abs(Fraction(float(y[i])) - ye) <= Fraction(k) * Fraction(2) ** -52 * Ae
        assert abs(Fraction(float(A[i])) - Ae) <= Fraction(k) * Fraction(2) ** -52 * Ae


def test_matvec_special_cases():
    w = S.normal_bf16(31, (37, 53), 0.02)
    for j in (0, 17, 52):
        x = np.zeros(53, np.uint16)
        x[j] = 0x3F80  # 1.0
        y, _ = O.matvec_bf16_ref(w, x)
        assert np.array_equal(y, O.bf16_value(w[:, j]))      # one-hot x picks column j
    eye = np.where(np.eye(40, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    x = S.activation_bf16(32, 40)
    y, _ = O.matvec_bf16_ref(eye, x)
    assert np.array_equal(y, O.bf16_value(x))
    # Small integers: every partial sum is an exact integer.
    rng = np.random.default_rng(33)
    wi = rng.integers(-20, 21, size=(16, 300)).astype(np.float32)
    xi = rng.integers(-20, 21, size=300).astype(np.float32)
    y, _ = O.matvec_bf16_ref(S.bf16_from_f32(wi), S.bf16_from_f32(xi))
    assert np.array_equal(y, wi.astype(np.int64) @ xi.astype(np.int64))


# --------------------------------------------------------------- gather
def test_gather_rows():
    w = S.normal_bf16(41, (300, 70), 0.02)
    enc = O.encode_bf16(w)
    ids = np.array([0, 299, 5, 5, 123, 299, -1, 300])
    g = O.gather_bf16_ref(enc, ids)
    assert np.array_equal(g[:6], w[ids[:6]])
    assert not g[6:].any()


# --------------------------------------------------------------- fp8
def test_fp8_values_match_torch():
    import torch
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.fp8_e4m3fn_value(b)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_fp8_all_bytes_roundtrip():
    q = S.all_bytes_fp8(4)
    enc = O.encode_fp8(q)
    assert np.array_equal(O.decode_fp8(enc), q)
    assert enc["coded_bits"] == O.coded_bits_closed_form_fp8(enc["counts"], enc["sym_to_rank"])


def test_fp8_single_matrix_roundtrip_size_and_quantisation():
    w = S.normal_bf16(C.SINGLE["w_seed"], (1024, 1024), C.SINGLE["sigma"])
    q, sc = S.fp8_quantize(w)
    enc = O.encode_fp8(q)
    rows = np.arange(0, 1024, 16)
    sub = dict(enc, n=len(rows), row_off=enc["row_off"][rows], row_bits=enc["row_bits"][rows])
    assert np.array_equal(O.decode_fp8(sub), q[rows])
    h = O.byte_entropy(q)
    assert q.size * h <= enc["coded_bits"]
    # The model card reports the coded fp8 at 0.87 of its bytes; the synthetic
    # Gaussian rows land below that (reported, not gated).
    assert enc["coded_bits"] / (8.0 * q.size) < 0.9
    # Quantisation: |q*s - w| is at most half an e4m3 step of the scaled value.
    wv = O.bf16_value(w)
    qv = O.fp8_e4m3fn_value(q)
    err = np.abs(qv * sc[:, None].astype(np.float64) - wv)
    assert np.all(err <= np.abs(wv) * 2.0 ** -4 + sc[:, None] * 2.0 ** -10 + 1e-30)


def test_fp8_matvec_exact_rationals():
    w = S.normal_bf16(51, (3, 200), 0.02)
    q, sc = S.fp8_quantize(w)
    x = S.activation_bf16(52, 200)
    y, A = O.matvec_fp8_ref(q, sc, x)
    qv = [Fraction(float(v)) for v in O.fp8_e4m3fn_value(q).reshape(-1)]
    X = _exact(x)
    for i in range(3):
        ye = Fraction(float(sc[i])) * sum(qv[i * 200 + j] * X[j] for j in range(200))
        Ae = abs(Fraction(float(sc[i]))) * sum(abs(qv[i * 200 + j] * X[j]) for j in range(200))
        assert abs(Fraction(float(y[i])) - ye) <= 200 * Fraction(2) ** -51 * Ae
        assert abs(Fraction(float(A[i])) - Ae) <= 200 * Fraction(2) ** -51 * Ae


def test_fp8_golden_bitstreams():
    ex = load_golden(GOLDEN_FP8, np.uint8)["C"]
    enc = O.encode_fp8(ex["w"])
    assert list(enc["rank_to_sym"][:len(ex["ranks"])]) == ex["ranks"]
    for r, bits in ex["rowbits"].items():
        off, nb = enc["row_off"][r], enc["row_bits"][r]
        assert list(enc["bits"][off:off + nb]) == bits
        # the same bits, codeword by codeword, from the codeword definition
        cw = []
        for b in ex["w"][r]:
            b = int(b)
            cw += O.codeword_fp8(int(enc["sym_to_rank"][(b >> 3) & 15]), b >> 7, (b >> 3) & 15, b & 7)
        assert cw == bits
    assert enc["coded_bits"] == ex["coded"]
    assert np.array_equal(O.decode_fp8(enc), ex["w"])


def test_fp8_kraft_and_prefix_free():
    # Symbol part (sign and the 3 raw mantissa bits excluded, both fixed-width):
    # ranks 0..7 are 1..8 bits, the 8 escaped fields 12 bits (8 ones + E).
    from fractions import Fraction
    r2s = np.arange(16)
    kraft = sum(Fraction(1, 2 ** (O.code_length_fp8(r) - 4)) for r in range(16))
    assert kraft == 1 - Fraction(1, 2 ** 8) + 8 * Fraction(1, 2 ** 12)
    assert kraft <= 1
    words = {}
    for b in range(256):
        s_, E, M = b >> 7, (b >> 3) & 15, b & 7
        w = tuple(O.codeword_fp8(int(np.where(r2s == E)[0][0]), s_, E, M))
        assert len(w) == O.code_length_fp8(E)
        assert w not in words
        words[w] = b
    ws = list(words)
    for a in ws:
        for c in ws:
            if a is not c:
                assert a != c[:len(a)], "fp8 codeword is a prefix of another"


def test_fp8_coded_bits_against_byte_entropy():
    # The whole-byte code against the byte's Shannon entropy on the fp8 copy of
    # the 1024 x 1024 matrix: above the bound (any prefix code is), and the
    # gap is what a code over whole bytes could still save (reported).
    w = S.normal_bf16(C.SINGLE["w_seed"], (1024, 1024), C.SINGLE["sigma"])
    q, _ = S.fp8_quantize(w)
    enc = O.encode_fp8(q)
    h = O.byte_entropy(q)
    per = enc["coded_bits"] / q.size
    print(f"fp8 1024x1024: H(byte) {h:.4f} bits, coded {per:.4f} bits ({per / h - 1:+.2%}), "
          f"{per / 8:.4f} of the fp8 bytes", flush=True)
    assert h <= per <= h + 1


# --------------------------------------------------------------- fp8 coder variant (length-limited Huffman)
GOLDEN_HUFF = os.path.join(os.path.dirname(__file__), "golden", "fp8_huffman_codes.txt")


def load_huffman_golden():
    ex = {"lengths": {}, "total": {}, "codes": {}, "row": {}, "rowbits": {}}
    for line in open(GOLDEN_HUFF):
        p = line.split()
        if not p or p[0].startswith("#"):
            continue
        if p[0] == "counts":
            ex["counts"] = {int(a, 16): int(b) for a, b in (t.split(":") for t in p[2:])}
        elif p[0] == "lengths":
            ex["lengths"][int(p[2])] = {int(a, 16): int(b) for a, b in (t.split(":") for t in p[3:])}
        elif p[0] == "total":
            ex["total"][int(p[2])] = int(p[3])
        elif p[0] == "codes":
            ex["codes"][int(p[2])] = {int(a, 16): [int(c) for c in b] for a, b in (t.split(":") for t in p[3:])}
        elif p[0] == "row":
            ex["row"][int(p[2])] = [int(v, 16) for v in p[3:]]
        elif p[0] == "rowbits":
            ex["rowbits"][int(p[2])] = [int(c) for c in p[3]]
    return ex


def test_huffman_golden_example():
    ex = load_huffman_golden()
    counts = np.zeros(256, np.int64)
    for s, c in ex["counts"].items():
        counts[s] = c
    for L, total in ex["total"].items():
        lengths = O.huffman_lengths_limited(counts, L)
        assert sum(int(counts[s]) * lengths[s] for s in range(256)) == total
        assert max(lengths) <= L and O.kraft_sum(lengths) <= 1
        if L in (3, 4):   # the optimal lengths are unique there (derivation in the file)
            assert {s: lengths[s] for s in ex["lengths"][L]} == ex["lengths"][L]
    for L, words in ex["codes"].items():
        codes = O.canonical_codes(O.huffman_lengths_limited(counts, L))
        assert {s: O.codeword_huffman(*codes[s]) for s in words} == words
    row = np.array([ex["row"][4]], dtype=np.uint8)
    enc = O.encode_fp8_huffman(row, max_len=4, filler_codeword=False)
    assert list(enc["bits"][:enc["row_bits"][0]]) == ex["rowbits"][4]
    assert enc["coded_bits"] == ex["total"][4]
    assert np.array_equal(O.decode_fp8_huffman(enc), row)


def test_huffman_lengths_optimal_bruteforce():
    # Every length vector of 1..L bits per symbol with Kraft sum <= 1 is a
    # prefix code (Kraft-McMillan); the package-merge lengths must reach the
    # smallest total among all of them.
    rng = np.random.default_rng(17)
    for trial in range(40):
        a = int(rng.integers(2, 7))
        counts = rng.integers(1, 60, size=a)
        for L in (max(1, int(np.ceil(np.log2(a)))), 3, 4, 6):
            if (1 << L) < a:
                continue
            got = O.huffman_lengths_limited(counts, L)
            best = min(sum(int(c) * l for c, l in zip(counts, ls))
                       for ls in itertools.product(range(1, L + 1), repeat=a)
                       if sum(Fraction(1, 2 ** l) for l in ls) <= 1)
            assert sum(int(c) * l for c, l in zip(counts, got)) == best, (counts, L, got)


def test_huffman_codes_prefix_free_and_complete():
    q, _ = S.fp8_quantize(S.normal_bf16(C.SINGLE["w_seed"], (1024, 1024), C.SINGLE["sigma"]))
    counts = np.bincount(q.reshape(-1), minlength=256)
    lengths = O.huffman_lengths_limited(counts)
    assert max(lengths) <= O.HUFF_MAX_LEN
    assert O.kraft_sum(lengths) == 1     # an optimal code with two or more symbols is complete
    words = [tuple(O.codeword_huffman(*cl)) for cl in O.canonical_codes(lengths).values()]
    for a in words:
        for b in words:
            if a is not b:
                assert a != b[:len(a)], "codeword is a prefix of another"


def test_huffman_fp8_size_against_entropy_and_the_unary_code():
    q, _ = S.fp8_quantize(S.normal_bf16(C.SINGLE["w_seed"], (1024, 1024), C.SINGLE["sigma"]))
    h = O.byte_entropy(q)
    huff = O.encode_fp8_huffman(q)
    unary = O.encode_fp8(q)
    per = huff["coded_bits"] / q.size
    print(f"fp8 1024x1024: H(byte) {h:.4f}, Huffman (<= 12 bits) {per:.4f} ({per / 8:.4f} of the bytes), "
          f"unary-rank code {unary['coded_bits'] / q.size:.4f}", flush=True)
    assert h <= per <= h + 1
    assert huff["coded_bits"] < unary["coded_bits"]
    assert np.array_equal(O.decode_fp8_huffman(huff), q)


def test_huffman_round_trips():
    for q in (S.all_bytes_fp8(3), np.full((3, 7), 0x38, np.uint8),
              S.fp8_quantize(S.odd_shape_matrix(1, "t3")[0])[0]):
        enc = O.encode_fp8_huffman(q)
        assert np.array_equal(O.decode_fp8_huffman(enc), q)
