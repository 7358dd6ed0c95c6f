"""Oracle pins on every generated matrix of the five workloads (CPU only).

The method is lossless ("neural-weight-compression 0.9.0" PyPI page, "How it
works": byte planes and a prefix code; "Qwen3-4B-NWC-fp8" model card: fp8
bytes recovered bit for bit), so the oracle's decode of its own encoding must
return every generated matrix bit for bit, and its coded size must sit between
the Shannon bound of the exponent/sign byte plus 8 raw mantissa bits and 2 %
above it.  These tests run the plain C oracle (oracle/nwc_oracle.c) over every
matrix the GPU tests and the benchmark use -- the same seeded host draws --
spread over the host's cores.  Its bits equal the numpy oracle's (checked in
test_oracle_c.py).
"""
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle as O
import synth as S
from oracle import fast as F
from synth import configs as C

THREADS = max(1, min(16, os.cpu_count() or 1))


def _entropy_gate(rt, nk):
    """N*K*(H(hi) + 8) <= coded <= 1.02 * N*K*(H(hi) + 8)."""
    c = rt["hi_counts"].astype(np.float64)
    p = c[c > 0] / c.sum()
    h = float(-(p * np.log2(p)).sum())
    lower = nk * (h + 8.0)
    return lower, rt["coded_bits"], rt["coded_bits"] / lower


def _check_matrix(m):
    w = S.blocked_normal_bf16(m["w_seed"], (m["n"], m["k"]), np.float32(m["sigma"]), threads=1)
    rt = F.roundtrip_bf16(w, threads=1)
    lower, coded, ratio = _entropy_gate(rt, w.size)
    return m["label"], rt["equal"], lower <= coded, ratio


def _run_all(mats, what):
    t0 = time.time()
    with ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(_check_matrix, mats))
    bad = [r for r in res if not (r[1] and r[2] and r[3] <= 1.02)]
    worst = max(res, key=lambda r: r[3])
    print(f"{what}: {len(res)} matrices round-tripped in {time.time() - t0:.1f}s on {THREADS} threads; "
          f"largest coded/(H+8) {worst[3]:.4f} ({worst[0]})", flush=True)
    assert not bad, f"{len(bad)} matrices failed: {bad[:5]}"
    return res


def test_single_matrix_every_bit_and_gate():
    w = S.normal_bf16(C.SINGLE["w_seed"], (C.SINGLE["n"], C.SINGLE["k"]), C.SINGLE["sigma"])
    rt = F.roundtrip_bf16(w)
    assert rt["equal"]
    lower, coded, ratio = _entropy_gate(rt, w.size)
    assert lower <= coded <= 1.02 * lower, ratio
    # The numpy oracle codes the same matrix to the same size.
    assert O.encode_bf16(w)["coded_bits"] == coded


def test_qwen3_4b_layer_set_every_matrix():
    res = _run_all(list(C.qwen3_matrices()), "qwen3_4b layer set")
    assert len(res) == C.QWEN3_4B_LAYERS * 7


def test_qwen25_7b_step_every_matrix():
    res = _run_all(list(C.qwen25_matrices()), "qwen25_7b step")
    assert len(res) == C.QWEN25_7B_LAYERS * 7 + 1


def test_tied_embedding_table_and_fp8_copy():
    res = _run_all([C.embedding_matrix()], "tied embedding")
    assert len(res) == 1
    q, scale = S.fp8_quantize(S.normal_bf16(C.SINGLE["w_seed"], (C.SINGLE["n"], C.SINGLE["k"]), C.SINGLE["sigma"]))
    rt = F.roundtrip_fp8(q)
    assert rt["equal"]
    assert rt["coded_bits"] == O.encode_fp8(q)["coded_bits"]


@pytest.mark.parametrize("idx", range(len(C.ODD_SHAPES)))
@pytest.mark.parametrize("kind", ["normal", "t3"])
def test_odd_shapes_every_matrix(idx, kind):
    w, _, _ = S.odd_shape_matrix(idx, kind)
    rt = F.roundtrip_bf16(w)
    assert rt["equal"]
    lower, coded, _ = _entropy_gate(rt, w.size)
    assert lower <= coded
    # The 2 % gate on the shapes whose injected rare values (0.1 %, at least
    # eight) do not dominate a tiny matrix.
    if w.size >= 100_000:
        assert coded <= 1.02 * lower


def test_all_patterns_matrix():
    w = S.all_patterns_bf16()
    rt = F.roundtrip_bf16(w)
    assert rt["equal"]
    # Every symbol occurs 512 times: ranks follow the symbols, and ranks >= 8 escape.
    assert list(rt["rank_to_sym"]) == list(range(128))
    assert rt["code_bits"] == 512 * (sum(r + 2 for r in range(8)) + 120 * 16)
