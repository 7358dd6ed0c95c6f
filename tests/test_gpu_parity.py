"""GPU parity of libnwc against the CPU oracle, through the C ABI.

Decode (dequant) and gather must be bit-exact; the matvec must satisfy
|y - y_ref| <= 1e-3 * sum_j |w_ij x_j| + 1e-6 per output, y_ref the oracle's
float64 sum.  Small workloads are checked element by element; every matrix of
the full-size workloads is checked on every element in test_gpu_workloads.py.
"""
import numpy as np
import pytest

import oracle as O
import synth as S
from synth import configs as C

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from decode_matvec_amd import nwc  # noqa: E402

DEV = "cuda"
RTOL, ATOL = 1e-3, 1e-6


def dev16(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def host16(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def run_matvec(dm, x_u16, scale=None):
    y = torch.full((dm.n,), float("nan"), dtype=torch.float32, device=DEV)
    dm.matvec(dev16(x_u16), y, scale=None if scale is None else torch.from_numpy(scale).to(DEV))
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def check_tol(y, y_ref, A, what=""):
    err = np.abs(y - y_ref)
    bad = ~(err <= RTOL * A + ATOL)
    assert not bad.any(), f"{what}: {bad.sum()} outputs out of tolerance, worst row {np.argmax(err - RTOL * A)}"


def dequant_host(dm, ld=None):
    ld = dm.k if ld is None else ld
    dt = torch.int16 if dm.elem == 0 else torch.uint8
    out = torch.full((dm.n, ld), -1, dtype=dt, device=DEV)
    dm.dequant(out, ld=ld)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    return (o.view(np.uint16) if dm.elem == 0 else o)[:, :dm.k]


def full_parity_bf16(w, x, cols=0, rows=0, check_matvec=True):
    print(f"case shape={w.shape} cols={cols} rows={rows}", flush=True)
    dm = nwc.DeviceMatrix(nwc.encode(w, cols_per_lane=cols, rows_per_wave=rows), DEV)
    enc = O.encode_bf16(w)
    assert np.array_equal(dequant_host(dm), O.decode_bf16(enc))
    if check_matvec:
        y_ref, A = O.matvec_bf16_ref(w, x)
        y = run_matvec(dm, x)
        check_tol(y, y_ref, A, f"{w.shape}")
        y2 = run_matvec(dm, x)
        assert np.array_equal(y, y2), "matvec not deterministic"
    return dm


# ----------------------------------------------------------------- single 1024 x 1024
# Work-item geometries (cols_per_lane, rows_per_wave): automatic; one lane per
# row with the row over 4 workgroups (span sums); 64 lanes per row in one
# wave; and the widths 32/48/64 with 8, 16 or 32 lanes per row.
GEOMETRIES = [(0, 0), (16, 64), (16, 1), (32, 8), (48, 4), (64, 2), (64, 16)]


@pytest.mark.parametrize("cols,rows", GEOMETRIES)
def test_single_matrix(cols, rows):
    w = S.normal_bf16(C.SINGLE["w_seed"], (1024, 1024), C.SINGLE["sigma"])
    x = S.activation_bf16(C.SINGLE["x_seed"], 1024)
    full_parity_bf16(w, x, cols, rows)


def test_row_over_two_workgroups():
    w = S.normal_bf16(41, (200, 66000), 0.02)
    x = S.activation_bf16(42, 66000)
    dm = full_parity_bf16(w, x, 64, 1)
    assert dm.info["n_spans"] == 2


def test_repeated_calls_and_graph_replays():
    # A persistent grid with more row groups than resident workgroups: calls in
    # a row and graph replays give the bits of the first call (the summation
    # order is fixed), and two matrices may share one workspace in a stream.
    w1 = S.normal_bf16(51, (9728, 2560), 0.02)
    w2 = S.normal_bf16(52, (200, 66000), 0.02)
    x1, x2 = S.activation_bf16(53, 2560), S.activation_bf16(54, 66000)
    d1 = nwc.DeviceMatrix(nwc.encode(w1), DEV)
    d2 = nwc.DeviceMatrix(nwc.encode(w2, cols_per_lane=64, rows_per_wave=1), DEV)
    assert d1.info["n_items"] // d1.info["waves_per_group"] > 2000 and d2.info["n_spans"] == 2
    t1, t2 = dev16(x1), dev16(x2)
    y1 = torch.empty(d1.n, dtype=torch.float32, device=DEV)
    y2 = torch.empty(d2.n, dtype=torch.float32, device=DEV)
    ws = torch.zeros(max(1, nwc.workspace_size(d2.header) // 4), dtype=torch.int32, device=DEV)
    nwc.matvec(d1.header, d1.d_blob, t1, y1, ws)
    nwc.matvec(d2.header, d2.d_blob, t2, y2, ws)
    torch.cuda.synchronize()
    ref1, ref2 = y1.cpu().numpy().copy(), y2.cpu().numpy().copy()
    y_ref, A = O.matvec_bf16_ref(w2, x2)
    check_tol(ref2.astype(np.float64), y_ref, A, "two spans")
    rows = np.unique(np.random.default_rng(55).integers(0, 9728, 200))
    y_ref, A = O.matvec_bf16_ref(w1[rows], x1)
    check_tol(ref1[rows].astype(np.float64), y_ref, A, "persistent grid")
    for _ in range(3):
        nwc.matvec(d1.header, d1.d_blob, t1, y1, ws)
        nwc.matvec(d2.header, d2.d_blob, t2, y2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(y1.cpu().numpy(), ref1) and np.array_equal(y2.cpu().numpy(), ref2)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nwc.matvec(d1.header, d1.d_blob, t1, y1, ws)
        nwc.matvec(d2.header, d2.d_blob, t2, y2, ws)
    for _ in range(3):
        y1.fill_(float("nan"))
        y2.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y1.cpu().numpy(), ref1) and np.array_equal(y2.cpu().numpy(), ref2)


def test_fillers_when_rank0_is_the_top_symbol():
    # Most weights have exponent symbol 0x7F, so rank 0 is 0x7F and a filler
    # (zero code bits, zero mantissa) decodes to 0x7F00 = 2^127: finite, and
    # times the zero activation past column K it must add exactly zero.
    rng = np.random.default_rng(43)
    n, k = 7, 513
    w = (0x7F00 | rng.integers(0, 0x80, size=(n, k)) | (rng.integers(0, 2, size=(n, k)) << 15)).astype(np.uint16)
    w[0, :5] = S.normal_bf16(44, (1, 5), 0.02)[0]
    x = S.bf16_from_f32((rng.standard_normal(k) * 1e-30).astype(np.float32))
    for cols, rows in ((0, 0), (32, 8), (64, 1)):
        dm = full_parity_bf16(w, x, cols, rows)
        assert dm.info["rank_to_sym"][0] == 0x7F


def test_dequant_row_pitch():
    w = S.normal_bf16(5, (130, 200), 0.02)
    dm = nwc.DeviceMatrix(nwc.encode(w), DEV)
    assert np.array_equal(dequant_host(dm, ld=216), w)


# ----------------------------------------------------------------- odd shapes, rare values
def _odd_cases():
    out = []
    for idx, (n, k) in enumerate(C.ODD_SHAPES):
        for kind in ("normal", "t3"):
            out.append((idx, n, k, kind))
    return out


@pytest.mark.parametrize("idx,n,k,kind", _odd_cases())
def test_odd_shapes(idx, n, k, kind):
    w, x, _ = S.odd_shape_matrix(idx, kind)
    full_parity_bf16(w, x)


def test_all_patterns_dequant_and_gather():
    w = S.all_patterns_bf16()
    dm = full_parity_bf16(w, None, check_matvec=False)
    ids = np.array([0, 255, 127, 128, 128, -3, 256, 1000, 7], dtype=np.int64)
    out = torch.full((len(ids), 256), -1, dtype=torch.int16, device=DEV)
    dm.gather(torch.from_numpy(ids).to(DEV), out)
    torch.cuda.synchronize()
    enc = O.encode_bf16(w)
    assert np.array_equal(host16(out), O.gather_bf16_ref(enc, ids))


def _gather_case(dm, expect_rows, ids, k, elem_u8=False):
    """nwc_gather of `ids`: each output row equals the expected row bit for bit (ids outside [0, n): zeros)."""
    dt = torch.uint8 if elem_u8 else torch.int16
    out = torch.full((len(ids), k), -1, dtype=dt, device=DEV)
    dm.gather(torch.from_numpy(ids).to(DEV), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    got = got if elem_u8 else got.view(np.uint16)
    assert np.array_equal(got, expect_rows), f"gather differs in rows {np.nonzero((got != expect_rows).any(1))[0][:8]}"


def _ids_for(n, seed, count=300):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, n, count).astype(np.int64)
    ids[:6] = [0, n - 1, -1, n, 1 << 40, ids[6]]  # ends, out of range on both sides, a duplicate
    return ids


@pytest.mark.parametrize("cols,rows", GEOMETRIES)
def test_gather_every_geometry(cols, rows):
    """Every work-item geometry, BF16 against the oracle's gather and fp8 against its definition."""
    print(f"case gather cols={cols} rows={rows}", flush=True)
    w = S.inject_rare(S.student_t_bf16(31, (1000, 1024)), 32)
    ids = _ids_for(1000, 33)
    dm = nwc.DeviceMatrix(nwc.encode(w, cols_per_lane=cols, rows_per_wave=rows), DEV)
    _gather_case(dm, O.gather_bf16_ref(O.encode_bf16(w), ids), ids, 1024)
    q, _ = S.fp8_quantize(w)
    dm8 = nwc.DeviceMatrix(nwc.encode(q, elem=nwc.NWC_FP8_E4M3, cols_per_lane=cols, rows_per_wave=rows), DEV)
    valid = (ids >= 0) & (ids < 1000)
    _gather_case(dm8, np.where(valid[:, None], q[np.clip(ids, 0, 999)], 0).astype(np.uint8), ids, 1024, True)


def test_gather_odd_shapes_and_split_rows():
    """Ragged K (last 16-column group partial), one-column rows, a row over two workgroups, one id."""
    for idx, (n, k, cols, rows) in enumerate(((7, 513, 0, 0), (1000, 3001, 0, 0), (4097, 1, 0, 0),
                                               (3, 65536, 0, 0), (200, 66000, 64, 1), (33, 257, 32, 32))):
        print(f"case gather shape={(n, k)}", flush=True)
        w = S.inject_rare(S.student_t_bf16(40 + idx, (n, k)), 50 + idx)
        dm = nwc.DeviceMatrix(nwc.encode(w, cols_per_lane=cols, rows_per_wave=rows), DEV)
        for ids in (_ids_for(n, 60 + idx, 97), np.array([n // 2], dtype=np.int64)):
            _gather_case(dm, O.gather_bf16_ref(O.encode_bf16(w), ids), ids, k)


# ----------------------------------------------------------------- exact special cases
def test_exact_special_cases():
    w = S.normal_bf16(31, (200, 300), 0.02)
    dm = nwc.DeviceMatrix(nwc.encode(w), DEV)
    for j in (0, 150, 299):
        x = np.zeros(300, np.uint16)
        x[j] = 0x3F80
        y_ref, _ = O.matvec_bf16_ref(w, x)
        assert np.array_equal(run_matvec(dm, x), y_ref)
    eye = np.where(np.eye(256, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    x = S.activation_bf16(32, 256)
    dm = nwc.DeviceMatrix(nwc.encode(eye), DEV)
    assert np.array_equal(run_matvec(dm, x), O.matvec_bf16_ref(eye, x)[0])
    rng = np.random.default_rng(33)
    wi = S.bf16_from_f32(rng.integers(-20, 21, size=(300, 1000)).astype(np.float32))
    xi = S.bf16_from_f32(rng.integers(-20, 21, size=1000).astype(np.float32))
    dm = nwc.DeviceMatrix(nwc.encode(wi), DEV)
    assert np.array_equal(run_matvec(dm, xi), O.matvec_bf16_ref(wi, xi)[0])


# ----------------------------------------------------------------- fp8 variant of the single matrix
# Both coders of the fp8 bytes: the pages' unary rank code and the
# length-limited Huffman variant (the same kernels decode both).
FP8_CODERS = [nwc.NWC_CODER_UNARY, nwc.NWC_CODER_HUFFMAN]


@pytest.mark.parametrize("coder", FP8_CODERS)
def test_fp8_single_matrix(coder):
    w = S.normal_bf16(C.SINGLE["w_seed"], (1024, 1024), C.SINGLE["sigma"])
    x = S.activation_bf16(C.SINGLE["x_seed"], 1024)
    q, sc = S.fp8_quantize(w)
    want = O.decode_fp8(O.encode_fp8(q)) if coder == nwc.NWC_CODER_UNARY else O.decode_fp8_huffman(
        O.encode_fp8_huffman(q))
    assert np.array_equal(want, q)
    for cols, rows in ((0, 0), (16, 64), (32, 8), (64, 1)):
        print(f"case fp8 coder={coder} cols={cols} rows={rows}", flush=True)
        dm = nwc.DeviceMatrix(nwc.encode(q, elem=nwc.NWC_FP8_E4M3, cols_per_lane=cols, rows_per_wave=rows,
                                         coder=coder), DEV)
        assert np.array_equal(dequant_host(dm), want)
        y_ref, A = O.matvec_fp8_ref(q, sc, x)
        check_tol(run_matvec(dm, x, sc), y_ref, A, "fp8")
        ids = np.array([0, 1023, 7, 7, 512], dtype=np.int64)
        out = torch.full((len(ids), 1024), 0xAB, dtype=torch.uint8, device=DEV)
        dm.gather(torch.from_numpy(ids).to(DEV), out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), q[ids])


@pytest.mark.parametrize("coder", FP8_CODERS)
def test_fp8_all_bytes_and_odd(coder):
    q = S.all_bytes_fp8(5)
    dm = nwc.DeviceMatrix(nwc.encode(q, elem=nwc.NWC_FP8_E4M3, coder=coder), DEV)
    assert np.array_equal(dequant_host(dm), q)
    w = S.inject_rare(S.student_t_bf16(71, (1000, 3001)), 72)
    q, sc = S.fp8_quantize(w)
    x = S.activation_bf16(73, 3001)
    dm = nwc.DeviceMatrix(nwc.encode(q, elem=nwc.NWC_FP8_E4M3, coder=coder), DEV)
    assert np.array_equal(dequant_host(dm), q)
    y_ref, A = O.matvec_fp8_ref(q, sc, x)
    check_tol(run_matvec(dm, x, sc), y_ref, A, "fp8 odd")


def test_fp8_huffman_full_size_and_one_value():
    # A Qwen3-4B gate-shaped fp8 matrix (9728 x 2560) under the Huffman
    # variant: every byte dequantized bit for bit, every output in tolerance;
    # and a matrix of one byte value, whose code is that byte plus the filler.
    w = S.blocked_normal_bf16(C.qwen3_seed(0, 4)[0], (9728, 2560), np.float32(C.sigma_for(2560)))
    q, sc = S.fp8_quantize(w)
    x = S.activation_bf16(C.qwen3_seed(0, 4)[1], 2560)
    dm = nwc.DeviceMatrix(nwc.encode(q, elem=nwc.NWC_FP8_E4M3, coder=nwc.NWC_CODER_HUFFMAN), DEV)
    assert np.array_equal(dequant_host(dm), q)
    from oracle import fast as F
    y_ref, A = F.matvec_fp8(q, sc, x)
    check_tol(run_matvec(dm, x, sc), y_ref, A, "fp8 huffman 9728x2560")
    q1 = np.full((33, 70), 0xB8, np.uint8)
    sc1 = np.ones(33, np.float32)
    x1 = S.activation_bf16(74, 70)
    d1 = nwc.DeviceMatrix(nwc.encode(q1, elem=nwc.NWC_FP8_E4M3, coder=nwc.NWC_CODER_HUFFMAN), DEV)
    assert np.array_equal(dequant_host(d1), q1)
    y_ref, A = O.matvec_fp8_ref(q1, sc1, x1)
    check_tol(run_matvec(d1, x1, sc1), y_ref, A, "fp8 huffman one value")


# ----------------------------------------------------------------- small batches
def _batch_case(dm, w, k, batch, seed, scale=None, q=None):
    """nwc_matvec_batch on `batch` activation rows (padded row pitches): every
    row equals nwc_matvec on that row bit for bit, nothing past a row's n
    outputs is written, and the first and last rows meet the oracle's bound."""
    ldx = (k + 7) // 8 * 8 + 8
    ldy = dm.n + 3
    xs = [S.activation_bf16(seed + b, k) for b in range(batch)]
    xh = np.zeros((batch, ldx), dtype=np.uint16)
    for b in range(batch):
        xh[b, :k] = xs[b]
    y = torch.full((batch, ldy), float("nan"), dtype=torch.float32, device=DEV)
    dm.matvec_batch(dev16(xh), y, scale=None if scale is None else torch.from_numpy(scale).to(DEV))
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.isnan(yh[:, dm.n:]).all(), "wrote past a row's outputs"
    for b in range(batch):
        assert np.array_equal(yh[b, :dm.n].astype(np.float64), run_matvec(dm, xs[b], scale)), f"row {b}"
    for b in sorted({0, batch - 1}):
        y_ref, A = O.matvec_bf16_ref(w, xs[b]) if q is None else O.matvec_fp8_ref(q, scale, xs[b])
        check_tol(yh[b, :dm.n].astype(np.float64), y_ref, A, f"batch row {b}")


@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 7])
def test_matvec_batch(batch):
    print(f"case batch={batch}", flush=True)
    w = S.normal_bf16(C.SINGLE["w_seed"], (1024, 1024), C.SINGLE["sigma"])
    for cols, rows in ((0, 0), (32, 4), (64, 2)):  # 16 and 32 columns per lane batched, 64 row by row
        dm = nwc.DeviceMatrix(nwc.encode(w, cols_per_lane=cols, rows_per_wave=rows), DEV)
        _batch_case(dm, w, 1024, batch, 600 + batch)


def test_matvec_batch_escapes_split_rows_and_fp8():
    w = S.inject_rare(S.student_t_bf16(81, (1000, 3001)), 82)  # long items decode from LDS
    _batch_case(nwc.DeviceMatrix(nwc.encode(w), DEV), w, 3001, 5, 700)
    w2 = S.normal_bf16(8, (200, 66000), 0.02)  # rows over two workgroups: one row at a time
    _batch_case(nwc.DeviceMatrix(nwc.encode(w2, cols_per_lane=64, rows_per_wave=1), DEV), w2, 66000, 3, 710)
    q, sc = S.fp8_quantize(S.normal_bf16(C.SINGLE["w_seed"], (1024, 1024), C.SINGLE["sigma"]))
    _batch_case(nwc.DeviceMatrix(nwc.encode(q, elem=nwc.NWC_FP8_E4M3), DEV), None, 1024, 3, 720, scale=sc, q=q)


# ----------------------------------------------------------------- prefill: dequantize + library GEMM
@pytest.mark.parametrize("tokens", [1, 7, 64])
def test_prefill_equals_the_library_gemm_on_the_weights(tokens):
    """Dequantization is exact, so prefill equals F.linear on the original BF16 weights bit for bit (same
    GEMM, same inputs); fp8 equals the widened e4m3 weights times the row scales.  Both also meet the
    oracle's bound widened by the GEMM's bf16 output rounding (2^-8 relative)."""
    import torch.nn.functional as F
    from decode_matvec_amd import prefill as P
    print(f"case prefill tokens={tokens}", flush=True)
    n, k = 1000, 3001
    w = S.student_t_bf16(91, (n, k))  # finite weights: outputs are compared with torch.equal
    X = np.stack([S.activation_bf16(900 + t, k) for t in range(tokens)])
    xt = dev16(X).view(torch.bfloat16)
    dm = nwc.DeviceMatrix(nwc.encode(w), DEV)
    y = P.prefill(dm, xt)
    assert y.dtype == torch.bfloat16 and tuple(y.shape) == (tokens, n)
    assert torch.equal(y, F.linear(xt, dev16(w).view(torch.bfloat16)))
    yh = y.float().cpu().numpy().astype(np.float64)
    for t in sorted({0, tokens - 1}):
        y_ref, A = O.matvec_bf16_ref(w, X[t])
        assert (np.abs(yh[t] - y_ref) <= 2.0 ** -8 * np.abs(y_ref) + RTOL * A + ATOL).all(), f"token {t}"
    q, sc = S.fp8_quantize(w)
    dm8 = nwc.DeviceMatrix(nwc.encode(q, elem=nwc.NWC_FP8_E4M3), DEV)
    scratch = torch.empty(n * k + 100, dtype=torch.uint8, device=DEV)  # larger than needed, reused
    s_d = torch.from_numpy(sc).to(DEV)
    wq = torch.from_numpy(q).to(DEV).view(torch.float8_e4m3fn).to(torch.bfloat16)
    want = (F.linear(xt, wq).float() * s_d[None, :]).to(torch.bfloat16)
    for _ in range(2):
        assert torch.equal(P.prefill(dm8, xt, scale=s_d, scratch=scratch), want)
    y8 = P.prefill(dm8, xt, scale=s_d).float().cpu().numpy().astype(np.float64)
    y_ref, A = O.matvec_fp8_ref(q, sc, X[0])
    assert (np.abs(y8[0] - y_ref) <= 2.0 ** -8 * np.abs(y_ref) + RTOL * A + ATOL).all()
    with pytest.raises(ValueError):
        P.prefill(dm8, xt)  # fp8 without its scales
    with pytest.raises(ValueError):
        P.prefill(dm, xt, scratch=scratch)  # BF16 needs an int16 buffer
    with pytest.raises(ValueError):
        P.prefill(dm, xt[:, :100])


# ----------------------------------------------------------------- uncompressed reference GEMV
@pytest.mark.parametrize("n,k,ld", [(300, 1000, 1000), (7, 24576, 24576), (33, 8, 16), (4097, 2560, 2568)])
def test_bf16_gemv_reference(n, k, ld):
    """The plain BF16 GEMV baseline meets the same bound against the oracle's float64 sum."""
    print(f"case bf16_gemv n={n} k={k} ld={ld}", flush=True)
    w = S.student_t_bf16(95, (n, k))
    x = S.activation_bf16(96, k)
    wp = np.zeros((n, ld), dtype=np.uint16)
    wp[:, :k] = w
    y = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    nwc.bf16_gemv(dev16(wp), dev16(x), y, k=k)
    torch.cuda.synchronize()
    y_ref, A = O.matvec_bf16_ref(w, x)
    check_tol(y.cpu().numpy().astype(np.float64), y_ref, A, "bf16 gemv")


# ----------------------------------------------------------------- full-size workloads
# Every matrix of the full-size workloads is checked element by element in
# test_gpu_workloads.py; here the decode step's wiring.


def test_qwen25_step_two_layers_matches_bf16_stack():
    # The decode step of the Qwen2.5-7B workload (two of its 28 layers plus the
    # lm_head) through nwc_matvec and through torch's BF16 linear, same glue:
    # every matrix is checked against the oracle elsewhere; this checks that
    # the step wiring (fp32 outputs, BF16 inputs, GQA stand-in) agrees.
    import bench
    stack, head, h0 = bench.build_qwen25_step(torch, nwc, S, C, DEV, 2, True, with_fused=True)
    F = torch.nn.functional

    def nwc_linear(m, x):
        m["dm"].matvec(x, m["y"])
        return m["y"]

    def bf16_linear(m, x):
        return F.linear(x.view(1, -1), m["w_bf16"]).view(-1).float()

    y_nwc = bench.qwen25_step(torch, stack, head, h0, nwc_linear).clone()
    y_fused = bench.qwen25_step(torch, stack, head, h0, nwc_linear, fused=True).clone()
    y_bf = bench.qwen25_step(torch, stack, head, h0, bf16_linear)
    torch.cuda.synchronize()
    assert torch.isfinite(y_nwc).all()
    rel = float((y_nwc - y_bf).norm() / y_bf.norm())
    rel_f = float((y_fused - y_nwc).norm() / y_nwc.norm())
    print(f"qwen2.5 two-layer step: logits rel L2 vs BF16 stack {rel:.2e}, fused vs separate {rel_f:.2e}", flush=True)
    assert rel < 1e-2
    # q||k||v and gate||up encoded as one matrix decode the same weights; only
    # the fp32 summation order of a row may differ.
    assert rel_f < 1e-4


def test_stream_read_helper():
    # The bandwidth reference reads any 16-byte multiple; a zero buffer folds to
    # zero, so the sink stays untouched.
    buf = torch.zeros(1 << 20, dtype=torch.int32, device=DEV)
    sink = torch.full((4,), 7, dtype=torch.int32, device=DEV)
    for nbytes in (16, 4096 + 16, buf.numel() * 4):
        nwc.stream_read(buf, sink, nbytes)
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [7, 7, 7, 7]


# ----------------------------------------------------------------- grouped launches
def test_matvec_group_mixed_shapes_fp8_and_graph_replays():
    # Twelve matrices of several work-item shapes (a launch per shape), fp8
    # members with their scales, and ragged shapes: each output bit-equal to
    # nwc_matvec on the same matrix and in tolerance against the oracle; calls
    # in a row and graph replays give the same bits.
    members = []
    for i, (n, k, cols, rows) in enumerate([(4096, 2560, 0, 0), (1024, 2560, 0, 0), (1000, 3001, 0, 0),
                                            (7, 513, 0, 0), (2560, 4096, 0, 0), (300, 1000, 32, 4),
                                            (300, 1000, 32, 4), (1023, 2560, 0, 0), (64, 64, 16, 64),
                                            (129, 700, 48, 2)]):
        w = S.normal_bf16(700 + i, (n, k), 0.02)
        x = S.activation_bf16(800 + i, k)
        members.append(dict(w=w, x=x, dm=nwc.DeviceMatrix(nwc.encode(w, cols_per_lane=cols, rows_per_wave=rows),
                                                          DEV), scale=None))
    for i in range(2):
        w = S.normal_bf16(900 + i, (1024, 1024), 0.02)
        q, sc = S.fp8_quantize(w)
        members.append(dict(q=q, sc=sc, x=S.activation_bf16(910 + i, 1024),
                            dm=nwc.DeviceMatrix(nwc.encode(q, elem=nwc.NWC_FP8_E4M3), DEV),
                            scale=torch.from_numpy(sc).to(DEV)))
    assert len(members) == nwc.GROUP_MAX
    xs = [dev16(m["x"]) for m in members]
    singles = []
    for m, x in zip(members, xs):
        y = torch.full((m["dm"].n,), float("nan"), dtype=torch.float32, device=DEV)
        m["dm"].matvec(x, y, scale=m["scale"])
        singles.append(y)
    ys = [torch.full_like(y, float("nan")) for y in singles]
    scales = [m["scale"] for m in members]
    nwc.matvec_group([m["dm"] for m in members], xs, ys, scales=scales)
    torch.cuda.synchronize()
    for m, y, y1 in zip(members, ys, singles):
        assert torch.equal(y, y1), "grouped output differs from nwc_matvec"
        if "w" in m:
            y_ref, A = O.matvec_bf16_ref(m["w"], m["x"])
        else:
            y_ref, A = O.matvec_fp8_ref(m["q"], m["sc"], m["x"])
        check_tol(y.cpu().numpy().astype(np.float64), y_ref, A, "group member")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nwc.matvec_group([m["dm"] for m in members], xs, ys, scales=scales)
    for _ in range(3):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(y, y1) for y, y1 in zip(ys, singles))


def test_bf16_gemv_group_reference():
    """The grouped plain BF16 GEMV baseline: every member within the bound of the oracle's float64 sum, and
    bit-equal to the single-matrix baseline."""
    shapes = [(4096, 2560, 2560), (1024, 2560, 2560), (1023, 2560, 2560), (7, 8, 16), (300, 9728, 9728),
              (5, 24576 + 8, 24576 + 8)]
    ws, xs, ys, ys1, refs = [], [], [], [], []
    for i, (n, k, ld) in enumerate(shapes):
        w = S.student_t_bf16(150 + i, (n, k))
        x = S.activation_bf16(160 + i, k)
        wp = np.zeros((n, ld), dtype=np.uint16)
        wp[:, :k] = w
        ws.append(dev16(wp)[:, :k] if ld != k else dev16(wp))
        xs.append(dev16(x))
        ys.append(torch.full((n,), float("nan"), dtype=torch.float32, device=DEV))
        y1 = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
        nwc.bf16_gemv(dev16(wp), dev16(x), y1, k=k)
        ys1.append(y1)
        refs.append(O.matvec_bf16_ref(w, x))
    nwc.bf16_gemv_group(ws, xs, ys)
    torch.cuda.synchronize()
    for y, y1, (y_ref, A) in zip(ys, ys1, refs):
        check_tol(y.cpu().numpy().astype(np.float64), y_ref, A, "bf16 gemv group")
        assert torch.equal(y, y1)


# ----------------------------------------------------------------- blob files on the device
def test_blob_file_round_trip_runs_every_kernel(tmp_path):
    # Encode, save to a blob file, load it back (host check of every blob) and
    # run the kernels on the loaded blobs: dequant and gather bit-exact and the
    # matvec (fp8 with the scales stored beside it) in tolerance against the
    # oracle -- no BF16 original is needed after the save.
    from decode_matvec_amd import store
    w = S.inject_rare(S.normal_bf16(171, (1000, 3001), 0.02), 172)
    q, sc = S.fp8_quantize(S.normal_bf16(173, (300, 2560), 0.02))
    path = str(tmp_path / "layer.safetensors")
    store.save(path, {"w": nwc.encode(w), "q": nwc.encode(q, elem=nwc.NWC_FP8_E4M3)}, {"q_scale": sc})
    blobs, arrays = store.load(path)
    dm = nwc.DeviceMatrix(blobs["w"], DEV)
    assert np.array_equal(dequant_host(dm), w)
    x = S.activation_bf16(174, 3001)
    y_ref, A = O.matvec_bf16_ref(w, x)
    check_tol(run_matvec(dm, x), y_ref, A, "loaded bf16 blob")
    ids = np.array([0, 999, 5, 5, 512], dtype=np.int64)
    out = torch.full((len(ids), 3001), -1, dtype=torch.int16, device=DEV)
    dm.gather(torch.from_numpy(ids).to(DEV), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w[ids])
    d8 = nwc.DeviceMatrix(blobs["q"], DEV)
    assert np.array_equal(dequant_host(d8), q)
    x8 = S.activation_bf16(175, 2560)
    y_ref, A = O.matvec_fp8_ref(q, arrays["q_scale"], x8)
    check_tol(run_matvec(d8, x8, scale=arrays["q_scale"]), y_ref, A, "loaded fp8 blob")


# ----------------------------------------------------------------- matrix-core small batches
@pytest.mark.parametrize("cols", [16, 32])
@pytest.mark.parametrize("batch", [5, 8, 16, 17, 32, 40])
def test_matvec_batch_matrix_cores(cols, batch):
    """Blobs of 16 rows per wave take the matrix-core path for 5 or more activation rows: every output of
    every row within the matvec bound of the oracle's float64 sum; the activations' padding past column k (NaN)
    is never used; nothing written past a row's outputs."""
    from oracle import fast as F
    cases = [("ragged with rare values", S.inject_rare(S.student_t_bf16(91, (1000, 3001)), 92)),
             ("q shape, rows over four spans", S.normal_bf16(93, (4096, 2560), float(np.float32(C.sigma_for(2560)))))]
    for what, w in cases:
        n, k = w.shape
        print(f"case mfma batch={batch} cols={cols} {what} {n}x{k}", flush=True)
        dm = nwc.DeviceMatrix(nwc.encode(w, cols_per_lane=cols, rows_per_wave=16), DEV)
        assert dm.info["rows_per_wave"] == 16 and dm.info["cols_per_lane"] == cols
        ldx = (k + 7) // 8 * 8 + 16
        ldy = n + 5
        xs = [S.activation_bf16(1000 * batch + b, k) for b in range(batch)]
        xh = np.full((batch, ldx), 0x7FC0, dtype=np.uint16)  # NaN past column k: must not be read
        for b in range(batch):
            xh[b, :k] = xs[b]
        y = torch.full((batch, ldy), float("nan"), dtype=torch.float32, device=DEV)
        dm.matvec_batch(dev16(xh), y)
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        assert np.isnan(yh[:, n:]).all(), "wrote past a row's outputs"
        for b in range(batch):
            y_ref, A = F.matvec_bf16(w, xs[b])
            check_tol(yh[b, :n].astype(np.float64), y_ref, A, f"{what}: row {b}")
