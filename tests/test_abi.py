"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
checks its arguments before touching the GPU, and its host encoder agrees with
the oracle (rank table, coded size, layout, decode table).  No GPU needed."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import synth as S
from synth import configs as C
from decode_matvec_amd import nwc

from . import blob_layout as BL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "nwc.h")).read()
    declared = set(re.findall(r"^(?:int|const char \*)\s*(nwc_\w+)\s*\(", hdr, re.M))
    assert declared == set(nwc.EXPORTS)
    lib = ctypes.CDLL(nwc.LIB_PATH)
    for name in declared:
        assert getattr(lib, name) is not None
    assert nwc.version() == 10000
    assert nwc.status_string(0) == "ok"
    assert "format" in nwc.status_string(-4)


def test_header_is_plain_c(tmp_path):
    """include/nwc.h is a C ABI: it compiles as strict C99 and as C++17, without warnings."""
    import shutil
    import subprocess
    src = tmp_path / "use.c"
    src.write_text('#include "nwc.h"\nint main(void) { nwc_info i; (void)i; return nwc_version() > 0 ? 0 : 1; }\n')
    inc = os.path.join(ROOT, "include")
    for cc, args in (("gcc", ["-std=c99", "-pedantic"]), ("g++", ["-std=c++17", "-x", "c++"])):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not installed")
        r = subprocess.run([cc, *args, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I", inc, str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def _mats():
    out = [("single", S.normal_bf16(1, (1024, 1024), 0.02)),
           ("all_patterns", S.all_patterns_bf16())]
    for idx, (n, k) in enumerate(C.ODD_SHAPES):
        out.append((f"odd{n}x{k}", S.inject_rare(S.student_t_bf16(C.odd_seed(2 * idx + 1), (n, k)),
                                                   C.odd_seed(2 * idx + 1) + 50)))
    return out


@pytest.mark.parametrize("name,w", _mats(), ids=lambda v: v if isinstance(v, str) else "")
def test_encoder_matches_oracle_rank_and_size(name, w):
    blob = nwc.encode(w)
    info = nwc.blob_info(blob)
    enc = O.encode_bf16(w)
    assert info["rank_to_sym"] == [int(v) for v in enc["rank_to_sym"]]
    assert info["coded_bits"] == enc["coded_bits"]
    assert (info["n"], info["k"]) == w.shape


def test_encoder_fp8_matches_oracle():
    q, _ = S.fp8_quantize(S.normal_bf16(1, (1024, 1024), 0.02))
    for m in (q, S.all_bytes_fp8(3)):
        blob = nwc.encode(m, elem=nwc.NWC_FP8_E4M3)
        info = nwc.blob_info(blob)
        enc = O.encode_fp8(m)
        assert info["rank_to_sym"][:16] == [int(v) for v in enc["rank_to_sym"]]
        assert info["coded_bits"] == enc["coded_bits"]


# (shape, cols_per_lane, rows_per_wave): automatic, every lane count per row
# (R = 64 .. 1), ragged K and N, and a row split over two workgroups.
@pytest.mark.parametrize("shape,cols,rows,seed", [((70, 333), 16, 8, 1), ((130, 100), 0, 0, 2), ((3, 600), 64, 1, 3),
                                                  ((64, 48), 16, 64, 4), ((9, 1000), 48, 2, 5), ((33, 257), 32, 32, 6),
                                                  ((2, 66000), 64, 1, 7)])
def test_blob_layout_decodes_to_input(shape, cols, rows, seed):
    w = S.inject_rare(S.student_t_bf16(seed, shape), seed + 7, frac=0.02)
    blob = nwc.encode(w, cols_per_lane=cols, rows_per_wave=rows)
    info = nwc.blob_info(blob)
    if cols:
        assert (info["cols_per_lane"], info["rows_per_wave"]) == (cols, rows)
    assert np.array_equal(BL.decode_blob(blob), w)
    q, _ = S.fp8_quantize(w)
    blob8 = nwc.encode(q, elem=nwc.NWC_FP8_E4M3, cols_per_lane=cols, rows_per_wave=rows)
    assert np.array_equal(BL.decode_blob(blob8), q)


def test_two_span_geometry():
    blob = nwc.encode(S.normal_bf16(8, (2, 66000), 0.02), cols_per_lane=64, rows_per_wave=1)
    info = nwc.blob_info(blob)
    # 1032 slices of 64 columns, 64 per wave: 17 waves, more than a workgroup holds.
    assert (info["n_spans"], info["waves_per_group"]) == (2, 9)
    assert info["n_items"] == 2 * 2 * 9


def test_matrix_core_geometry_keeps_two_workgroups_per_cu():
    # 16 rows per wave: at most 12 waves per workgroup (two fit under the 25-wave cap), the columns spread
    # over as few spans as that allows; 2 rows of each shape keep the encode cheap.
    for k, want in ((2560, (4, 10)), (4096, (6, 11)), (9728, (13, 12)), (1000, (2, 8))):
        info = nwc.blob_info(nwc.encode(S.normal_bf16(k, (2, k), 0.02), cols_per_lane=16, rows_per_wave=16))
        assert (info["n_spans"], info["waves_per_group"]) == want, k
        assert info["n_spans"] * info["waves_per_group"] * 4 * 16 >= k
    # other explicit geometries keep up to 16 waves
    info = nwc.blob_info(nwc.encode(S.normal_bf16(9, (2, 4096), 0.02), cols_per_lane=16, rows_per_wave=4))
    assert (info["n_spans"], info["waves_per_group"]) == (1, 16)


def test_auto_geometry_of_the_layer_shapes():
    # Every Qwen3-4B projection gets a geometry whose row group fits one
    # workgroup (no span sums), stores at most 6% filler columns (K = 9728 =
    # 19*512 pads 5.3% in every geometry that fits), and whose
    # double-buffered workgroup fits 64 KiB of LDS.
    for n, k in [(1024, 2560), (4096, 2560), (2560, 4096), (9728, 2560), (2560, 9728)]:
        info = nwc.blob_info(nwc.encode(S.normal_bf16(1, (n, k), 0.02)))
        C, R, W = info["cols_per_lane"], info["rows_per_wave"], info["waves_per_group"]
        assert info["n_spans"] == 1, (n, k)
        lane_cols = -(-n // R) * R * W * (64 // R) * C
        assert lane_cols <= 1.06 * n * k, (n, k, C, R, W)
        assert 2 * (W * (info["max_rows"] + 2) * 256 + W * R * 4) + 16384 <= 65536


def test_all_patterns_blob_layout():
    w = S.all_patterns_bf16()
    assert np.array_equal(BL.decode_blob(nwc.encode(w)), w)


def test_decode_table_bf16_against_oracle():
    w = S.normal_bf16(9, (300, 500), 0.02)
    blob = nwc.encode(w)
    r2s = np.array(BL.header(blob)["rank_to_sym"], dtype=np.int64)
    lut = BL.lut(blob)
    for p in range(4096):
        bits = [(p >> i) & 1 for i in range(12)]
        e = int(lut[p])
        # Oracle parse of the two leading codes, if both end inside the 12 bits.
        pad = bits + [0] * 32
        sa, ea, pa = O.parse_one_bf16(pad, 0, r2s)
        ok = pa <= 12 and sum(bits[:8]) < 8 or False
        if ok and not (pa == 16):
            sb, eb, pb = O.parse_one_bf16(pad, pa, r2s)
            ok = pb <= 12 and pb - pa != 16
        if ok:
            assert e == pb | (((sa << 7) | ea) << 8) | (((sb << 7) | eb) << 16), p
        else:
            assert e == 0x80000000, p


def test_decode_table_fp8_against_oracle():
    q, _ = S.fp8_quantize(S.normal_bf16(1, (256, 256), 0.02))
    blob = nwc.encode(q, elem=nwc.NWC_FP8_E4M3)
    lut = BL.lut(blob)
    h = BL.header(blob)
    import torch
    for p in range(4096):
        e = int(lut[p])
        bits = [(p >> i) & 1 for i in range(12)]
        if all(bits[:8]):
            assert e == 0x80000000
            continue
        r = bits.index(0)
        s = bits[r + 1]
        M = bits[r + 2] | bits[r + 3] << 1 | bits[r + 4] << 2
        E = h["rank_to_sym"][r]
        b = (s << 7) | (E << 3) | M
        bf = torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.bfloat16)
        want = int(bf.view(torch.int16).item()) & 0xFFFF
        if torch.isnan(bf).item():   # torch canonicalises the NaN sign; any BF16 NaN will do
            assert (e & 0x7F80) == 0x7F80 and (e & 0x7F) != 0
        else:
            assert e & 0xFFFF == want
        assert (e >> 16) & 0xFF == b and (e >> 24) == r + 5


def test_encoder_argument_errors():
    w = np.zeros((4, 8), np.uint16)
    blob = np.zeros(1 << 20, np.uint8)
    size = ctypes.c_int64()
    L = nwc.lib
    enc = lambda *a: L.nwc_encode(*a, blob.ctypes.data, blob.nbytes, ctypes.byref(size))
    assert enc(None, 4, 8, 8, 0, 0, 0) == -1
    assert enc(w.ctypes.data, 4, 8, 8, 7, 0, 0) == -1      # element type
    assert enc(w.ctypes.data, 4, 8, 4, 0, 0, 0) == -2      # ld < k
    assert enc(w.ctypes.data, 0, 8, 8, 0, 0, 0) == -2
    assert enc(w.ctypes.data, 4, 8, 8, 0, 24, 0) == -1     # cols_per_lane not a multiple of 16
    assert enc(w.ctypes.data, 4, 8, 8, 0, 128, 0) == -1    # cols_per_lane too large
    assert enc(w.ctypes.data, 4, 8, 8, 0, 0, 6) == -1      # rows_per_wave not a power of two
    assert enc(w.ctypes.data, 4, 8, 8, 0, 0, 128) == -1
    assert L.nwc_encode(w.ctypes.data, 4, 8, 8, 0, 0, 0, blob.ctypes.data, 100, ctypes.byref(size)) == -3
    assert enc(w.ctypes.data, 4, 8, 8, 0, 0, 0) == 0
    with pytest.raises(TypeError):
        nwc.encode(w.astype(np.float32))


def test_bound_covers_worst_case():
    # The all-escape matrix (every symbol ties) is the longest code there is.
    w = S.all_patterns_bf16()
    assert nwc.encode(w).nbytes <= nwc.encode_bound(256, 256)
    for cols in (16, 32, 64):
        for rows in (1, 8, 64):
            assert nwc.encode(w, cols_per_lane=cols, rows_per_wave=rows).nbytes <= \
                nwc.encode_bound(256, 256, 0, cols, rows)


def _two_span():
    w = S.normal_bf16(3, (200, 66000), 0.02)
    return w, nwc.encode(w, cols_per_lane=64, rows_per_wave=1)


def test_header_validation_and_workspace():
    w, blob = _two_span()
    hdr = blob[:256].copy()
    info = nwc.blob_info(blob)
    assert info["n_spans"] == 2
    assert nwc.workspace_size(hdr) == ((200 * 4 * 4 + 255) // 256) * 256   # [row][span padded to 4] fp32
    bad = hdr.copy()
    bad[0] ^= 1
    with pytest.raises(nwc.NWCError) as ei:
        nwc.workspace_size(bad)
    assert ei.value.status == -4
    bad = hdr.copy()
    bad[8] = 5  # elem
    with pytest.raises(nwc.NWCError):
        nwc.blob_info(np.concatenate([bad, blob[256:]]))
    bad = hdr.copy()
    bad[36] = 3  # rows_per_wave not a power of two
    with pytest.raises(nwc.NWCError):
        nwc.workspace_size(bad)
    # A row held by one workgroup needs no workspace.
    assert nwc.workspace_size(nwc.encode(S.normal_bf16(3, (70, 100), 0.02))[:256].copy()) == 0


def test_launchers_reject_bad_arguments_before_any_gpu_call():
    w, blob = _two_span()
    hdr = blob[:256].copy()
    L = nwc.lib
    fake = 1 << 20  # never dereferenced: every call below fails its host-side checks
    ws = nwc.workspace_size(hdr)
    assert L.nwc_matvec(None, fake, fake, None, fake, fake, ws, None) == -1
    assert L.nwc_matvec(hdr.ctypes.data, 0, fake, None, fake, fake, ws, None) == -1
    assert L.nwc_matvec(hdr.ctypes.data, fake + 4, fake, None, fake, fake, ws, None) == -1
    assert L.nwc_matvec(hdr.ctypes.data, fake, fake, fake, fake, fake, ws, None) == -1   # BF16 with a scale
    assert L.nwc_matvec(hdr.ctypes.data, fake, fake, None, fake, None, ws, None) == -1   # workspace missing
    assert L.nwc_matvec(hdr.ctypes.data, fake, fake, None, fake, fake, ws - 4, None) == -3
    bad = hdr.copy()
    bad[4] = 9  # version
    assert L.nwc_matvec(bad.ctypes.data, fake, fake, None, fake, fake, ws, None) == -4
    # nwc_matvec_batch(header, blob, x, ldx, batch, scale, y, ldy, ws, ws_bytes, stream)
    assert L.nwc_matvec_batch(hdr.ctypes.data, fake, fake, 66000, -1, None, fake, 200, fake, ws, None) == -2
    assert L.nwc_matvec_batch(hdr.ctypes.data, fake, fake, 65992, 3, None, fake, 200, fake, ws, None) == -2  # ldx < k
    assert L.nwc_matvec_batch(hdr.ctypes.data, fake, fake, 66004, 3, None, fake, 200, fake, ws, None) == -2  # ldx % 8
    assert L.nwc_matvec_batch(hdr.ctypes.data, fake, fake, 66000, 3, None, fake, 199, fake, ws, None) == -2  # ldy < n
    assert L.nwc_matvec_batch(hdr.ctypes.data, fake, 0, 66000, 3, None, fake, 200, fake, ws, None) == -1
    assert L.nwc_matvec_batch(hdr.ctypes.data, fake, fake, 66000, 3, None, fake + 2, 200, fake, ws, None) == -1
    assert L.nwc_matvec_batch(hdr.ctypes.data, fake, fake, 66000, 3, fake, fake, 200, fake, ws, None) == -1
    assert L.nwc_matvec_batch(bad.ctypes.data, fake, fake, 66000, 3, None, fake, 200, fake, ws, None) == -4
    assert L.nwc_matvec_batch(hdr.ctypes.data, fake, fake, 66000, 0, None, fake, 200, fake, ws, None) == 0
    assert L.nwc_dequant(hdr.ctypes.data, fake, fake, 65999, None) == -2
    assert L.nwc_dequant(hdr.ctypes.data, fake, fake + 2, 66000, None) == -1
    assert L.nwc_gather(hdr.ctypes.data, fake, fake, -1, fake, None) == -2
    assert L.nwc_gather(hdr.ctypes.data, fake, fake + 4, 5, fake, None) == -1
    assert L.nwc_gather(hdr.ctypes.data, fake, fake, 0, fake, None) == 0   # nothing to do
    assert L.nwc_stream_read(None, 1024, fake, None) == -1
    assert L.nwc_stream_read(fake + 8, 1024, fake, None) == -1
    assert L.nwc_stream_read(fake, 1000, fake, None) == -2
    assert L.nwc_stream_read(fake, 0, fake, None) == 0   # nothing to read
    q, _ = S.fp8_quantize(S.normal_bf16(3, (200, 700), 0.02))
    h8 = nwc.encode(q, elem=1)[:256].copy()
    assert L.nwc_matvec(h8.ctypes.data, fake, fake, None, fake, None, 0, None) == -1   # fp8 needs a scale


def test_bf16_gemv_rejects_bad_arguments_before_any_gpu_call():
    L = ctypes.CDLL(nwc.LIB_PATH)
    L.nwc_bf16_gemv.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p]
    fake = 1 << 20  # aligned, never dereferenced: every call below fails its checks first
    assert L.nwc_bf16_gemv(None, 4, 64, 64, fake, fake, None) == -1
    assert L.nwc_bf16_gemv(fake + 8, 4, 64, 64, fake, fake, None) == -1       # w not 16-byte aligned
    assert L.nwc_bf16_gemv(fake, 4, 60, 64, fake, fake, None) == -2           # k not a multiple of 8
    assert L.nwc_bf16_gemv(fake, 4, 64, 56, fake, fake, None) == -2           # ldw < k
    assert L.nwc_bf16_gemv(fake, 4, 64, 60, fake, fake, None) == -2           # ldw not a multiple of 8
    assert L.nwc_bf16_gemv(fake, 0, 64, 64, fake, fake, None) == -2


def test_bf16_gemv_group_rejects_bad_arguments_before_any_gpu_call():
    L = nwc.lib
    fake = 1 << 20
    ok = (fake, 4, 64, 64, fake, fake)

    def descs(*rows):
        arr = (nwc.GemvDesc * max(1, len(rows)))()
        for i, r in enumerate(rows):
            arr[i] = nwc.GemvDesc(*r)
        return arr

    assert L.nwc_bf16_gemv_group(descs(ok), 0, None) == 0
    assert L.nwc_bf16_gemv_group(descs(*[ok] * 13), 13, None) == -2
    assert L.nwc_bf16_gemv_group(None, 1, None) == -1
    assert L.nwc_bf16_gemv_group(descs(ok, (fake + 8, 4, 64, 64, fake, fake)), 2, None) == -1
    assert L.nwc_bf16_gemv_group(descs(ok, (fake, 4, 60, 64, fake, fake)), 2, None) == -2
    assert L.nwc_bf16_gemv_group(descs(ok, (fake, 0, 64, 64, fake, fake)), 2, None) == -2


def test_one_hip_runtime_whatever_the_import_order():
    # Loading the library before torch once put two HIP runtimes in the process
    # (PyTorch's bundled one and /opt/rocm's); the library's then saw no device.
    import subprocess
    import sys
    code = ("from decode_matvec_amd import nwc\nimport torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "print(sorted({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    paths = eval(out.stdout.strip().splitlines()[-1])
    assert len(paths) == 1, paths


class _FakeDev:
    """Stands in for a device tensor in host-side argument checks (never dereferenced)."""

    def __init__(self, numel, esize, floating=False, contiguous=True, cuda=True):
        import torch
        self._n, self._e, self.is_cuda, self._c = numel, esize, cuda, contiguous
        self.dtype = {(4, True): torch.float32, (4, False): torch.int32, (2, False): torch.int16,
                      (2, True): torch.bfloat16, (1, False): torch.uint8, (8, False): torch.int64}[(esize, floating)]

    def numel(self):
        return self._n

    def element_size(self):
        return self._e

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        raise AssertionError("the binding passed a rejected tensor on to the library")


def test_binding_checks_tensor_arguments_on_the_host():
    w = S.normal_bf16(5, (70, 100), 0.02)
    hdr = nwc.encode(w)[:256].copy()
    blob = _FakeDev(1 << 20, 1)
    ok_x, ok_y = _FakeDev(100, 2), _FakeDev(70, 4, True)
    bad = [("x short", _FakeDev(99, 2), ok_y), ("x 4-byte", _FakeDev(100, 4, True), ok_y),
           ("x on host", _FakeDev(100, 2, cuda=False), ok_y), ("x strided", _FakeDev(100, 2, contiguous=False), ok_y),
           ("y short", ok_x, _FakeDev(69, 4, True)), ("y int", ok_x, _FakeDev(70, 4, False)),
           ("y bf16", ok_x, _FakeDev(70, 2, True))]
    for what, x, y in bad:
        with pytest.raises(ValueError):
            nwc.matvec(hdr, blob, x, y)
    with pytest.raises(ValueError):   # dequant output too small for (n-1)*ld + k elements
        nwc.dequant(hdr, blob, _FakeDev(69 * 128 + 99, 2), 128)
    with pytest.raises(ValueError):   # ld < k
        nwc.dequant(hdr, blob, _FakeDev(70 * 128, 2), 99)
    with pytest.raises(ValueError):   # fp8 bytes expected for an fp8 blob, not BF16
        q, _ = S.fp8_quantize(w)
        nwc.dequant(nwc.encode(q, elem=1)[:256].copy(), blob, _FakeDev(70 * 100, 2), 100)
    with pytest.raises(ValueError):   # ids must be int64
        nwc.gather(hdr, blob, _FakeDev(4, 4, False), _FakeDev(400, 2))
    ids = _FakeDev(4, 8)
    with pytest.raises(ValueError):   # out must hold n_ids * k elements
        nwc.gather(hdr, blob, ids, _FakeDev(399, 2))
    q, _ = S.fp8_quantize(w)
    h8 = nwc.encode(q, elem=1)[:256].copy()
    with pytest.raises(ValueError):   # fp8 needs n fp32 scales
        nwc.matvec(h8, blob, ok_x, ok_y, scale=_FakeDev(69, 4, True))


def test_matvec_group_rejects_bad_arguments_before_any_gpu_call():
    L = nwc.lib
    fake = 1 << 20  # aligned, never dereferenced: every call below fails its host-side checks first
    w = S.normal_bf16(5, (70, 100), 0.02)
    hdr = nwc.encode(w)[:256].copy()
    _, two = _two_span()
    hdr2 = two[:256].copy()

    def descs(*rows):
        arr = (nwc.MatvecDesc * max(1, len(rows)))()
        for i, r in enumerate(rows):
            arr[i] = nwc.MatvecDesc(*r)
        return arr

    ok = (hdr.ctypes.data, fake, fake, None, fake)
    assert L.nwc_matvec_group(descs(ok), 0, None) == 0                       # nothing to do
    assert L.nwc_matvec_group(descs(ok), -1, None) == -2
    assert L.nwc_matvec_group(descs(*[ok] * 13), 13, None) == -2             # more than NWC_GROUP_MAX
    assert L.nwc_matvec_group(None, 2, None) == -1
    assert L.nwc_matvec_group(descs(ok, (hdr.ctypes.data, fake, fake + 4, None, fake)), 2, None) == -1  # x misaligned
    assert L.nwc_matvec_group(descs(ok, (hdr.ctypes.data, fake, fake, fake, fake)), 2, None) == -1      # BF16 + scale
    assert L.nwc_matvec_group(descs(ok, (None, fake, fake, None, fake)), 2, None) == -1
    bad = hdr.copy()
    bad[4] = 9
    assert L.nwc_matvec_group(descs(ok, (bad.ctypes.data, fake, fake, None, fake)), 2, None) == -4
    assert L.nwc_matvec_group(descs(ok, (hdr2.ctypes.data, fake, fake, None, fake)), 2, None) == -6     # split rows
    q, _ = S.fp8_quantize(w)
    h8 = nwc.encode(q, elem=1)[:256].copy()
    assert L.nwc_matvec_group(descs(ok, (h8.ctypes.data, fake, fake, None, fake)), 2, None) == -1       # fp8, no scale


def _grown_header(hdr, n):
    """A valid header of the same geometry for n rows (dependent fields recomputed; never launched)."""
    h = np.frombuffer(hdr.tobytes(), dtype=BL.HDR)[0].copy()
    R, W, sp = int(h["rows_per_wave"]), int(h["waves_per_group"]), int(h["n_spans"])
    h["n"] = n
    h["n_rowgroups"] = (n + R - 1) // R
    h["n_items"] = int(h["n_rowgroups"]) * sp * W
    h["off_mant"] = int(h["off_items"]) + (int(h["n_items"]) * 8 + 255) // 256 * 256
    h["mant_bytes"] = int(h["n_items"]) * 64 * int(h["cols_per_lane"])
    h["off_code"] = int(h["off_mant"]) + int(h["mant_bytes"])
    h["code_bytes"] = int(h["n_items"]) * 256
    h["total_bytes"] = int(h["off_code"]) + int(h["code_bytes"])
    return np.frombuffer(h.tobytes(), dtype=np.uint8).copy()


def test_matvec_noalloc_rejects_bad_arguments_before_any_gpu_call():
    L = nwc.lib
    fake = 1 << 20
    _, blob = _two_span()
    hdr = blob[:256].copy()
    assert nwc.workspace_size(hdr) <= nwc.NOALLOC_SCRATCH_BYTES
    assert L.nwc_matvec_noalloc(None, fake, fake, None, fake, None) == -1
    assert L.nwc_matvec_noalloc(hdr.ctypes.data, 0, fake, None, fake, None) == -1
    assert L.nwc_matvec_noalloc(hdr.ctypes.data, fake, fake + 4, None, fake, None) == -1
    assert L.nwc_matvec_noalloc(hdr.ctypes.data, fake, fake, fake, fake, None) == -1     # BF16 with a scale
    bad = hdr.copy()
    bad[4] = 9
    assert L.nwc_matvec_noalloc(bad.ctypes.data, fake, fake, None, fake, None) == -4
    # Partials beyond the static scratch: refused with a capacity error, nothing enqueued.
    big = _grown_header(hdr, 300000)
    assert nwc.workspace_size(big) > nwc.NOALLOC_SCRATCH_BYTES
    assert L.nwc_matvec_noalloc(big.ctypes.data, fake, fake, None, fake, None) == -3
    fits = _grown_header(hdr, 200000)
    assert nwc.workspace_size(fits) <= nwc.NOALLOC_SCRATCH_BYTES


# ----------------------------------------------------------------- Huffman coder variant (fp8 bytes)
def _fp8_mats():
    q1, _ = S.fp8_quantize(S.normal_bf16(C.SINGLE["w_seed"], (C.SINGLE["n"], C.SINGLE["k"]), C.SINGLE["sigma"]))
    qt, _ = S.fp8_quantize(S.odd_shape_matrix(1, "t3")[0])
    qz = np.full((5, 40), 0x38, np.uint8)   # one byte value: 0x00 added as the filler codeword
    return [("single_1024", q1), ("t3_1000x3001", qt), ("all_bytes", S.all_bytes_fp8(3)), ("one_value", qz)]


@pytest.mark.parametrize("name,q", _fp8_mats(), ids=lambda v: v if isinstance(v, str) else "")
def test_huffman_encoder_size_equals_the_oracle_optimum(name, q):
    blob = nwc.encode(q, elem=nwc.NWC_FP8_E4M3, coder=nwc.NWC_CODER_HUFFMAN)
    info = nwc.blob_info(blob)
    assert info["coder"] == nwc.NWC_CODER_HUFFMAN
    lengths = BL.huffman_lengths(BL.header(blob))
    assert max(lengths) <= 12 and lengths[0] > 0 and O.kraft_sum(lengths) <= 1
    counts = np.bincount(q.reshape(-1), minlength=256)
    assert all(lengths[b] > 0 for b in range(256) if counts[b])
    # Optimal length-limited codes have one total size: the library's package-merge and the oracle's agree.
    enc = O.encode_fp8_huffman(q)
    assert info["coded_bits"] == enc["coded_bits"] == int((counts * np.array(lengths)).sum())
    nwc.blob_check(blob)


@pytest.mark.parametrize("shape,cols,rows,seed", [((70, 333), 16, 8, 1), ((130, 100), 0, 0, 2), ((3, 600), 64, 1, 3),
                                                  ((9, 1000), 48, 2, 5), ((2, 66000), 64, 1, 7)])
def test_huffman_blob_layout_decodes_to_input(shape, cols, rows, seed):
    q, _ = S.fp8_quantize(S.inject_rare(S.student_t_bf16(seed, shape), seed + 7, frac=0.02))
    blob = nwc.encode(q, elem=nwc.NWC_FP8_E4M3, cols_per_lane=cols, rows_per_wave=rows, coder=nwc.NWC_CODER_HUFFMAN)
    assert np.array_equal(BL.decode_blob(blob), q)


def test_decode_table_huffman_against_oracle():
    q, _ = S.fp8_quantize(S.normal_bf16(1, (256, 256), 0.02))
    blob = nwc.encode(q, elem=nwc.NWC_FP8_E4M3, coder=nwc.NWC_CODER_HUFFMAN)
    lut = BL.lut(blob)
    codes = O.canonical_codes(BL.huffman_lengths(BL.header(blob)))
    import torch
    hits = 0
    for b, (c, l) in codes.items():
        bits = O.codeword_huffman(c, l)
        first = sum(v << i for i, v in enumerate(bits))   # stream order, first bit at bit 0
        bf = torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.bfloat16)
        want_bf = int(bf.view(torch.int16).item()) & 0xFFFF
        for p in range(first, 4096, 1 << l):
            e = int(lut[p])
            if torch.isnan(bf).item():
                assert (e & 0x7F80) == 0x7F80 and (e & 0x7F) != 0
            else:
                assert e & 0xFFFF == want_bf
            assert (e >> 16) & 0xFF == b and (e >> 24) == l
            hits += 1
    assert hits == 4096   # a complete code: every 12-bit peek starts exactly one codeword


def test_huffman_blob_check_rejects_bad_lengths():
    q, _ = S.fp8_quantize(S.normal_bf16(2, (64, 300), 0.02))
    blob = nwc.encode(q, elem=nwc.NWC_FP8_E4M3, coder=nwc.NWC_CODER_HUFFMAN)
    nwc.blob_check(blob)
    h = BL.header(blob)
    lengths = BL.huffman_lengths(h)
    used = [b for b in range(256) if lengths[b]]

    def with_lengths(ls):
        bad = blob.copy()
        for i in range(128):
            bad[128 + i] = (ls[2 * i] & 15) | (ls[2 * i + 1] << 4)
        return bad

    ls = list(lengths)
    ls[used[-1]] = 13                      # longer than the 12-bit peek
    with pytest.raises(nwc.NWCError):
        nwc.blob_check(with_lengths(ls))
    ls = list(lengths)
    ls[0] = 0                              # no filler codeword
    with pytest.raises(nwc.NWCError):
        nwc.blob_check(with_lengths(ls))
    ls = list(lengths)
    ls[[b for b in range(256) if not lengths[b]][0]] = 1    # Kraft sum above one
    with pytest.raises(nwc.NWCError):
        nwc.blob_check(with_lengths(ls))
    ls = list(lengths)
    a, b = used[1], used[2]
    ls[a], ls[b] = ls[b], ls[a]            # a valid code, but not the one the decode table holds
    if ls != lengths:
        with pytest.raises(nwc.NWCError):
            nwc.blob_check(with_lengths(ls))
    with pytest.raises(nwc.NWCError):      # Huffman only for fp8
        nwc.encode(S.normal_bf16(2, (4, 8), 0.02), coder=nwc.NWC_CODER_HUFFMAN)
