"""ctypes wrapper of the plain C oracle (oracle/nwc_oracle.c) for full-size workloads.

TEST INFRASTRUCTURE ONLY (see the package docstring).  The C file computes what
oracle/nwc_ref.py computes -- one bit stream per row, codes in column order,
float64 row sums -- in scalar C, so that every generated matrix of the
workloads (billions of weights) can be round-tripped and every matvec output
checked in minutes.  This module only marshals arrays, splits matrices into
row blocks (which does not change any result: every row is coded, decoded and
summed on its own, under the one per-matrix rank table) and runs blocks on
threads (ctypes releases the GIL during a call).

The library is built by ``build()`` (gcc) and, if it is missing when first
used, built on the spot.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nwc_oracle.c")
LIB_PATH = os.path.join(HERE, "libnwc_oracle.so")

ROW_BLOCK_WEIGHTS = 1 << 22  # weights per row block (memory only; results do not depend on it)


def build(verbose: bool = False) -> str:
    """Compile oracle/nwc_oracle.c into oracle/libnwc_oracle.so with gcc."""
    cc = os.environ.get("CC", "gcc")
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed ({r.returncode}):\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        sig = {
            "nwc_oracle_rank_table": ([vp, ci, vp, vp], None),
            "nwc_oracle_bf16_histogram": ([vp, i64, i64, i64, vp], None),
            "nwc_oracle_bf16_hi_histogram": ([vp, i64, i64, i64, vp], None),
            "nwc_oracle_bf16_encode": ([vp, i64, i64, i64, vp, vp, i64, vp], i64),
            "nwc_oracle_bf16_decode": ([vp, vp, i64, i64, vp, vp, i64, vp, i64], ci),
            "nwc_oracle_bf16_matvec": ([vp, i64, i64, i64, vp, vp, vp], None),
            "nwc_oracle_fp8_histogram": ([vp, i64, i64, i64, vp], None),
            "nwc_oracle_fp8_encode": ([vp, i64, i64, i64, vp, vp, i64, vp], i64),
            "nwc_oracle_fp8_decode": ([vp, vp, i64, i64, vp, vp, i64], ci),
            "nwc_oracle_fp8_matvec": ([vp, i64, i64, i64, vp, vp, vp, vp], None),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def _rows(w: np.ndarray):
    if w.ndim != 2 or w.strides[1] != w.itemsize:
        raise ValueError("expected a 2-D array with unit column stride")
    return w.shape[0], w.shape[1], w.strides[0] // w.itemsize


def _blocks(n: int, k: int):
    rb = max(1, ROW_BLOCK_WEIGHTS // max(k, 1))
    return [(r, min(n, r + rb)) for r in range(0, n, rb)]


def _pool(threads):
    return ThreadPoolExecutor(max(1, threads or os.cpu_count() or 1))


def rank_table(counts):
    counts = np.ascontiguousarray(counts, dtype=np.uint64)
    a = len(counts)
    r2s = np.zeros(a, np.uint8)
    s2r = np.zeros(a, np.uint8)
    lib().nwc_oracle_rank_table(_p(counts), a, _p(r2s), _p(s2r))
    return r2s, s2r


def _histogram(fn, w, bins, threads):
    n, k, ld = _rows(w)

    def one(b):
        c = np.zeros(bins, np.uint64)
        fn(_p(w[b[0]:b[1]]), b[1] - b[0], k, ld, _p(c))
        return c

    with _pool(threads) as ex:
        return sum(ex.map(one, _blocks(n, k)))


def bf16_histogram(w, threads=None):
    """Counts of the 7-bit exponent symbol (w >> 8) & 0x7F."""
    return _histogram(lib().nwc_oracle_bf16_histogram, w, 128, threads)


def bf16_hi_histogram(w, threads=None):
    """Counts of the whole high byte (sign and exponent symbol)."""
    return _histogram(lib().nwc_oracle_bf16_hi_histogram, w, 256, threads)


def encode_rows_bf16(w, sym_to_rank):
    """Bit streams of the rows of w: (stream uint64 words, row_start[n + 1] bit offsets, total bits)."""
    n, k, ld = _rows(w)
    words = (16 * n * k + 63) // 64 + 1
    stream = np.zeros(words, np.uint64)
    start = np.zeros(n + 1, np.int64)
    s2r = np.ascontiguousarray(sym_to_rank, dtype=np.uint8)
    bits = lib().nwc_oracle_bf16_encode(_p(w), n, k, ld, _p(s2r), _p(stream), words, _p(start))
    if bits < 0:
        raise RuntimeError("oracle stream overflow")
    return stream, start, int(bits)


def decode_rows_bf16(stream, start, n, k, rank_to_sym, mant):
    out = np.empty((n, k), np.uint16)
    r2s = np.ascontiguousarray(rank_to_sym, dtype=np.uint8)
    mant = np.ascontiguousarray(mant, dtype=np.uint8)
    st = lib().nwc_oracle_bf16_decode(_p(stream), _p(start), n, k, _p(r2s), _p(mant), k, _p(out), k)
    if st != 0:
        raise RuntimeError("oracle stream does not decode to its recorded length")
    return out


def roundtrip_bf16(w, threads=None) -> dict:
    """Encode every row of w under the matrix's rank table, decode it from its
    stream and its raw mantissa bytes, and compare with w.

    Returns counts (7-bit symbols), hi_counts (whole high byte), rank_to_sym,
    code_bits (sum of codeword lengths), coded_bits (+ 8 raw bits per weight)
    and ``equal`` (every decoded row equals its input, bit for bit)."""
    n, k, _ = _rows(w)
    counts = bf16_histogram(w, threads)
    hi = bf16_hi_histogram(w, threads)
    r2s, s2r = rank_table(counts)

    def one(b):
        blk = w[b[0]:b[1]]
        stream, start, bits = encode_rows_bf16(blk, s2r)
        mant = (blk & 0xFF).astype(np.uint8)
        dec = decode_rows_bf16(stream, start, b[1] - b[0], k, r2s, mant)
        return bits, bool(np.array_equal(dec, blk))

    with _pool(threads) as ex:
        res = list(ex.map(one, _blocks(n, k)))
    code_bits = sum(r[0] for r in res)
    return dict(counts=counts, hi_counts=hi, rank_to_sym=r2s, code_bits=code_bits,
                coded_bits=code_bits + 8 * n * k, equal=all(r[1] for r in res))


def matvec_bf16(w, x, threads=None):
    """(y, A) in float64: y_i = sum_j w_ij x_j, A_i = sum_j |w_ij x_j|."""
    n, k, ld = _rows(w)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    if x.size != k:
        raise ValueError("x must have k elements")
    y = np.empty(n, np.float64)
    a = np.empty(n, np.float64)

    def one(b):
        lib().nwc_oracle_bf16_matvec(_p(w[b[0]:b[1]]), b[1] - b[0], k, ld, _p(x), _p(y[b[0]:]), _p(a[b[0]:]))

    with _pool(threads) as ex:
        list(ex.map(one, _blocks(n, k)))
    return y, a


def fp8_histogram(q, threads=None):
    return _histogram(lib().nwc_oracle_fp8_histogram, q, 16, threads)


def roundtrip_fp8(q, threads=None) -> dict:
    """As roundtrip_bf16 for fp8 e4m3fn bytes coded whole (the byte is in the stream)."""
    n, k, ld = _rows(q)
    counts = fp8_histogram(q, threads)
    r2s, s2r = rank_table(counts)

    def one(b):
        blk = q[b[0]:b[1]]
        nb = b[1] - b[0]
        words = (16 * nb * k + 63) // 64 + 1
        stream = np.zeros(words, np.uint64)
        start = np.zeros(nb + 1, np.int64)
        bits = lib().nwc_oracle_fp8_encode(_p(blk), nb, k, ld, _p(s2r), _p(stream), words, _p(start))
        if bits < 0:
            raise RuntimeError("oracle stream overflow")
        out = np.empty((nb, k), np.uint8)
        if lib().nwc_oracle_fp8_decode(_p(stream), _p(start), nb, k, _p(r2s), _p(out), k) != 0:
            raise RuntimeError("oracle stream does not decode to its recorded length")
        return int(bits), bool(np.array_equal(out, blk))

    with _pool(threads) as ex:
        res = list(ex.map(one, _blocks(n, k)))
    code_bits = sum(r[0] for r in res)
    return dict(counts=counts, rank_to_sym=r2s, code_bits=code_bits, coded_bits=code_bits,
                equal=all(r[1] for r in res))


def matvec_fp8(q, scale, x, threads=None):
    """(y, A): y_i = s_i * sum_j q_ij x_j in float64, A_i = |s_i| * sum_j |q_ij x_j|."""
    n, k, ld = _rows(q)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    y = np.empty(n, np.float64)
    a = np.empty(n, np.float64)

    def one(b):
        lib().nwc_oracle_fp8_matvec(_p(q[b[0]:b[1]]), b[1] - b[0], k, ld, _p(scale[b[0]:]), _p(x), _p(y[b[0]:]),
                                    _p(a[b[0]:]))

    with _pool(threads) as ex:
        list(ex.map(one, _blocks(n, k)))
    return y, a
