"""Pins of the plain C oracle (oracle/nwc_oracle.c) -- CPU only.

The C oracle is what checks the full-size workloads, so it is pinned on its
own against the same fixed facts as the numpy oracle: the hand-derived worked
examples in tests/golden/, the all-patterns matrix, closed-form code lengths,
exact rational matvec sums and special cases.  It must also write the numpy
oracle's bits exactly (two independent writings of one definition).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth as S
from oracle import fast as F
from .test_oracle import GOLDEN_FP8, load_golden


def _bits(stream, start, r):
    """Bits of row r of a C-oracle stream, in stream order."""
    return [int((int(stream[p >> 6]) >> (p & 63)) & 1) for p in range(int(start[r]), int(start[r + 1]))]


@pytest.mark.parametrize("name", ["A", "B"])
def test_golden_bitstreams(name):
    ex = load_golden()[name]
    w = ex["w"]
    counts = F.bf16_histogram(w)
    r2s, s2r = F.rank_table(counts)
    assert list(r2s[:len(ex["ranks"])]) == ex["ranks"]
    stream, start, bits = F.encode_rows_bf16(w, s2r)
    for r, want in ex["rowbits"].items():
        assert _bits(stream, start, r) == want
    assert bits + 8 * w.size == ex["coded"]
    dec = F.decode_rows_bf16(stream, start, w.shape[0], w.shape[1], r2s, (w & 0xFF).astype(np.uint8))
    assert np.array_equal(dec, w)


def test_fp8_golden_bitstreams():
    ex = load_golden(GOLDEN_FP8, np.uint8)["C"]
    q = ex["w"]
    r2s, s2r = F.rank_table(F.fp8_histogram(q))
    assert list(r2s[:len(ex["ranks"])]) == ex["ranks"]
    n, k = q.shape
    words = (16 * n * k + 63) // 64 + 1
    stream = np.zeros(words, np.uint64)
    start = np.zeros(n + 1, np.int64)
    bits = F.lib().nwc_oracle_fp8_encode(q.ctypes.data, n, k, k, s2r.ctypes.data, stream.ctypes.data, words,
                                         start.ctypes.data)
    assert bits == ex["coded"]
    for r, want in ex["rowbits"].items():
        assert _bits(stream, start, r) == want
    assert F.roundtrip_fp8(q)["equal"]


def test_rank_table_ties_and_order():
    rng = np.random.default_rng(3)
    for _ in range(50):
        a = int(rng.choice([16, 128]))
        counts = rng.integers(0, 4, size=a)       # many ties
        r2s, s2r = F.rank_table(counts)
        o_r2s, o_s2r = O.rank_table(counts)
        assert list(r2s) == list(o_r2s) and list(s2r) == list(o_s2r)


def _cases():
    out = [("all_patterns", S.all_patterns_bf16())]
    for idx in range(3):
        for kind in ("normal", "t3"):
            w, _, _ = S.odd_shape_matrix(idx, kind)
            out.append((f"odd{idx}_{kind}", w[:200]))
    out.append(("rare_dense", S.inject_rare(S.normal_bf16(9, (40, 300), 0.02), 10, frac=0.2)))
    return out


@pytest.mark.parametrize("name,w", _cases(), ids=lambda v: v if isinstance(v, str) else "")
def test_same_bits_as_the_numpy_oracle(name, w):
    enc = O.encode_bf16(w)
    counts = F.bf16_histogram(w)
    assert np.array_equal(counts.astype(np.int64), enc["counts"])
    r2s, s2r = F.rank_table(counts)
    stream, start, bits = F.encode_rows_bf16(w, s2r)
    assert bits + 8 * w.size == enc["coded_bits"]
    assert bits + 8 * w.size == O.coded_bits_closed_form_bf16(enc["counts"], enc["sym_to_rank"], w.size)
    for r in range(w.shape[0]):
        off, nb = enc["row_off"][r], enc["row_bits"][r]
        assert _bits(stream, start, r) == list(enc["bits"][off:off + nb])
    assert F.roundtrip_bf16(w)["equal"]


def test_fp8_same_bits_as_the_numpy_oracle():
    q = np.concatenate([S.all_bytes_fp8(2), S.fp8_quantize(S.normal_bf16(4, (30, 256), 0.02))[0]])
    enc = O.encode_fp8(q)
    rt = F.roundtrip_fp8(q)
    assert rt["equal"] and rt["code_bits"] == enc["coded_bits"]


def test_decoder_rejects_a_stream_of_the_wrong_length():
    w = S.normal_bf16(5, (3, 40), 0.02)
    r2s, s2r = F.rank_table(F.bf16_histogram(w))
    stream, start, bits = F.encode_rows_bf16(w, s2r)
    bad = start.copy()
    bad[1] += 1   # row 0 claims one more bit than its codes use
    with pytest.raises(RuntimeError):
        F.decode_rows_bf16(stream, bad, 3, 40, r2s, (w & 0xFF).astype(np.uint8))


def _exact(u16):
    return [Fraction(float(v)) for v in S.f32_from_bf16(u16).reshape(-1)]


@pytest.mark.parametrize("n,k,seed", [(1, 1, 1), (3, 17, 2), (4, 600, 3)])
def test_matvec_against_exact_rationals(n, k, seed):
    w = S.normal_bf16(seed, (n, k), 0.5)
    x = S.activation_bf16(seed + 100, k)
    y, A = F.matvec_bf16(w, x)
    W, X = _exact(w), _exact(x)
    for i in range(n):
        ye = sum(W[i * k + j] * X[j] for j in range(k))
        Ae = sum(abs(W[i * k + j] * X[j]) for j in range(k))
        assert abs(Fraction(float(y[i])) - ye) <= k * Fraction(2) ** -52 * Ae
        assert abs(Fraction(float(A[i])) - Ae) <= k * Fraction(2) ** -52 * Ae


def test_matvec_special_cases():
    w = S.normal_bf16(7, (50, 64), 0.02)
    onehot = np.zeros(64, np.uint16)
    onehot[9] = 0x3F80    # 1.0
    y, _ = F.matvec_bf16(w, onehot)
    assert np.array_equal(y, O.bf16_value(w[:, 9]))
    eye = np.where(np.eye(64, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    x = S.activation_bf16(8, 64)
    y, A = F.matvec_bf16(eye, x)
    assert np.array_equal(y, O.bf16_value(x)) and np.array_equal(A, np.abs(O.bf16_value(x)))


def test_fp8_matvec_against_exact_rationals():
    w = S.normal_bf16(51, (3, 200), 0.02)
    q, sc = S.fp8_quantize(w)
    x = S.activation_bf16(52, 200)
    y, A = F.matvec_fp8(q, sc, x)
    qv = [Fraction(float(v)) for v in O.fp8_e4m3fn_value(q).reshape(-1)]
    X = _exact(x)
    for i in range(3):
        ye = Fraction(float(sc[i])) * sum(qv[i * 200 + j] * X[j] for j in range(200))
        assert abs(Fraction(float(y[i])) - ye) <= 200 * Fraction(2) ** -51 * abs(ye + 1)
    y2, A2 = O.matvec_fp8_ref(q, sc, x)
    assert np.allclose(y, y2, rtol=0, atol=1e-12) and np.allclose(A, A2, rtol=0, atol=1e-12)
