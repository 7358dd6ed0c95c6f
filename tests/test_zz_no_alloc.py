"""nwc_matvec_noalloc against nwc_matvec through the C ABI (GPU).

The entry point that allocates nothing keeps the span partials of split-row
matrices in the library's static per-GPU scratch.  Two calls in a row, the
second on a smaller matrix (so the scratch holds the first call's partials
when the second starts), must each give nwc_matvec's bits exactly, and every
output must be within |y - y_ref| <= 1e-3 sum_j |w_ij x_j| + 1e-6 of the
oracle's float64 sums.
"""
import ctypes

import numpy as np
import pytest

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from decode_matvec_amd import nwc  # noqa: E402

DEV = "cuda"


def _dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def _case(seed, n, k, cols, rows):
    w = S.normal_bf16(seed, (n, k), 0.02)
    x = S.activation_bf16(seed + 1, k)
    dm = nwc.DeviceMatrix(nwc.encode(w, cols_per_lane=cols, rows_per_wave=rows), DEV)
    return w, x, dm


def _noalloc_c(dm, xd, y, scale=None):
    # straight through the C ABI (the binding adds only host checks)
    st = nwc.lib.nwc_matvec_noalloc(dm.header.ctypes.data, dm.d_blob.data_ptr(), xd.data_ptr(),
                                    None if scale is None else scale.data_ptr(), y.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert st == 0, nwc.status_string(st)


def _check(w, x, dm, y_no, what):
    xd = _dev16(x)
    y_ref_dev = torch.full((dm.n,), float("nan"), dtype=torch.float32, device=DEV)
    dm.matvec(xd, y_ref_dev)
    torch.cuda.synchronize()
    assert torch.equal(y_no, y_ref_dev), f"{what}: nwc_matvec_noalloc differs from nwc_matvec"
    y_ref, A = O.matvec_bf16_ref(w, x)
    err = np.abs(y_no.cpu().numpy().astype(np.float64) - y_ref)
    assert np.all(err <= 1e-3 * A + 1e-6), f"{what}: outputs out of tolerance"


def test_noalloc_two_calls_second_smaller():
    # 16 columns per lane, one row per wave: a row longer than 16*64*16 =
    # 16384 columns spans two workgroups, so both matrices use the scratch.
    w1, x1, d1 = _case(61, 300, 20000, 16, 1)
    w2, x2, d2 = _case(62, 90, 17000, 16, 1)
    assert d1.info["n_spans"] == 2 and d2.info["n_spans"] == 2
    assert nwc.workspace_size(d2.header) < nwc.workspace_size(d1.header) <= nwc.NOALLOC_SCRATCH_BYTES
    print("case noalloc 300x20000 then 90x17000", flush=True)
    y1 = torch.full((d1.n,), float("nan"), dtype=torch.float32, device=DEV)
    y2 = torch.full((d2.n,), float("nan"), dtype=torch.float32, device=DEV)
    _noalloc_c(d1, _dev16(x1), y1)
    _noalloc_c(d2, _dev16(x2), y2)
    torch.cuda.synchronize()
    _check(w1, x1, d1, y1, "first call")
    _check(w2, x2, d2, y2, "second, smaller call")


def test_noalloc_rows_in_one_workgroup_and_fp8():
    # No split rows: no scratch is touched; fp8 with its scales.
    w, x, dm = _case(63, 257, 3001, 0, 0)
    assert dm.info["n_spans"] == 1
    y = torch.full((dm.n,), float("nan"), dtype=torch.float32, device=DEV)
    nwc.matvec_noalloc(dm.header, dm.d_blob, _dev16(x), y)
    torch.cuda.synchronize()
    _check(w, x, dm, y, "one span")
    q, sc = S.fp8_quantize(S.normal_bf16(64, (200, 20000), 0.02))
    d8 = nwc.DeviceMatrix(nwc.encode(q, elem=nwc.NWC_FP8_E4M3, cols_per_lane=16, rows_per_wave=1), DEV)
    assert d8.info["n_spans"] == 2
    xs = S.activation_bf16(65, 20000)
    sct = torch.from_numpy(sc).to(DEV)
    y8 = torch.full((200,), float("nan"), dtype=torch.float32, device=DEV)
    y8r = torch.full((200,), float("nan"), dtype=torch.float32, device=DEV)
    _noalloc_c(d8, _dev16(xs), y8, sct)
    d8.matvec(_dev16(xs), y8r, scale=sct)
    torch.cuda.synchronize()
    assert torch.equal(y8, y8r)
    y_ref, A = O.matvec_fp8_ref(q, sc, xs)
    assert np.all(np.abs(y8.cpu().numpy().astype(np.float64) - y_ref) <= 1e-3 * A + 1e-6)
