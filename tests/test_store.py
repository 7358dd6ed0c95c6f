"""CPU tests of the full blob check (nwc_blob_check) and of blob files
(decode_matvec_amd.store): valid blobs pass, every kind of damage that could
steer a kernel's memory accesses or decode is rejected, and a saved file loads
back to the same bytes, which still decode to the input matrix."""
import numpy as np
import pytest

import synth as S
from decode_matvec_amd import nwc, store

from . import blob_layout as BL

OFF_ITEMS = 256 + 16384  # header, then the 4096-entry decode table
OFF_LUT = 256
OFF_RANK = 128


def _blobs():
    w = S.inject_rare(S.student_t_bf16(11, (70, 333)), 18, frac=0.02)
    q, sc = S.fp8_quantize(w)
    return w, q, sc, {"bf16": nwc.encode(w, cols_per_lane=16, rows_per_wave=8),
                      "fp8": nwc.encode(q, elem=nwc.NWC_FP8_E4M3),
                      "two_span": nwc.encode(S.normal_bf16(8, (2, 66000), 0.02), cols_per_lane=64, rows_per_wave=1)}


def _status(blob):
    try:
        nwc.blob_check(blob)
    except nwc.NWCError as e:
        return e.status
    return 0


def _u32(blob, off):
    return int(np.frombuffer(blob[off:off + 4].tobytes(), "<u4")[0])


def _put_u32(blob, off, v):
    blob[off:off + 4] = np.frombuffer(np.uint32(v).tobytes(), np.uint8)


def test_check_accepts_encoded_blobs():
    *_, blobs = _blobs()
    for b in blobs.values():
        assert _status(b) == 0
    # Trailing bytes after the blob are allowed (blob_bytes is what is available).
    assert _status(np.concatenate([blobs["bf16"], np.zeros(100, np.uint8)])) == 0


def test_check_rejects_damage():
    *_, blobs = _blobs()
    b0 = blobs["bf16"]
    info = nwc.blob_info(b0)
    code_bytes, max_rows, n_items = info["code_bytes"], info["max_rows"], info["n_items"]
    last = OFF_ITEMS + 8 * (n_items - 1)

    def damaged(fn):
        b = b0.copy()
        fn(b)
        return _status(b)

    assert _status(b0[:-1]) == -3                                        # shorter than total_bytes
    assert _status(b0[:100]) == -3                                       # not even a header
    assert damaged(lambda b: b.__setitem__(0, b[0] ^ 1)) == -4           # magic
    assert damaged(lambda b: _put_u32(b, last, code_bytes)) == -4        # item code past the plane
    assert damaged(lambda b: _put_u32(b, last, _u32(b, last) + 4)) == -4  # not on a 256-byte row
    assert damaged(lambda b: _put_u32(b, last + 4, max_rows + 1)) == -4  # longer than max_rows
    assert damaged(lambda b: _put_u32(b, OFF_ITEMS + 4, 0)) == -4        # no rows
    assert damaged(lambda b: _put_u32(b, OFF_ITEMS, 0xFFFFFF00)) == -4   # offset far outside
    assert damaged(lambda b: b.__setitem__(OFF_LUT + 4 * 5, b[OFF_LUT + 4 * 5] ^ 1)) == -4  # table entry length
    assert damaged(lambda b: b.__setitem__(OFF_RANK + 1, b[OFF_RANK])) == -4  # symbol ranked twice
    # A swap of two ranks is a valid rank table but not the one the stored decode table was built from.
    def swap(b):
        b[OFF_RANK], b[OFF_RANK + 1] = b[OFF_RANK + 1], b[OFF_RANK]
    assert damaged(swap) == -4
    b8 = blobs["fp8"].copy()
    b8[OFF_RANK + 3] = 16                                                # fp8 exponent field out of range
    assert _status(b8) == -4


def test_save_load_round_trip(tmp_path):
    w, q, sc, blobs = _blobs()
    path = str(tmp_path / "m.safetensors")
    store.save(path, blobs, {"fp8.scale": sc, "norm": np.arange(5, dtype=np.float32)})
    got, arrays = store.load(path)
    assert sorted(got) == sorted(blobs)
    for k in blobs:
        assert np.array_equal(got[k], blobs[k])
    assert np.array_equal(arrays["fp8.scale"], sc) and arrays["fp8.scale"].dtype == sc.dtype
    assert np.array_equal(arrays["norm"], np.arange(5, dtype=np.float32))
    assert np.array_equal(BL.decode_blob(got["bf16"]), w)
    assert np.array_equal(BL.decode_blob(got["fp8"]), q)


def test_load_rejects_damaged_or_foreign_files(tmp_path):
    from safetensors.numpy import save_file

    *_, blobs = _blobs()
    bad = blobs["bf16"].copy()
    _put_u32(bad, OFF_ITEMS + 4, 10_000)
    path = str(tmp_path / "bad.safetensors")
    save_file({"w": bad}, path, metadata={"format": store.FORMAT, "blobs": "w"})
    with pytest.raises(nwc.NWCError):
        store.load(path)
    path = str(tmp_path / "foreign.safetensors")
    save_file({"w": blobs["bf16"]}, path)
    with pytest.raises(ValueError):
        store.load(path)
    path = str(tmp_path / "missing.safetensors")
    save_file({"w": blobs["bf16"]}, path, metadata={"format": store.FORMAT, "blobs": "w,v"})
    with pytest.raises(ValueError):
        store.load(path)
    with pytest.raises(nwc.NWCError):
        store.save(str(tmp_path / "x.safetensors"), {"w": bad})
    with pytest.raises(ValueError):
        store.save(str(tmp_path / "x.safetensors"), {"w": blobs["bf16"]}, {"w": np.zeros(1)})
