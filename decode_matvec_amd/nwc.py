"""Thin Python binding of libnwc (argument marshalling only).

Every step of the hot path runs in the HIP library; this module only converts
numpy arrays and torch tensors to pointers and sizes, and raises on error
statuses.  torch is used for device memory and streams.  Importing this
module fails loudly if the built library is missing: there is no fallback.

Function names mirror the C ABI in include/nwc.h.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnwc.so")

NWC_BF16 = 0
NWC_FP8_E4M3 = 1
NWC_CODER_UNARY = 0
NWC_CODER_HUFFMAN = 1
HEADER_BYTES = 256
GROUP_MAX = 12

STATUS = {0: "NWC_OK", -1: "NWC_ERR_ARG", -2: "NWC_ERR_SHAPE", -3: "NWC_ERR_CAPACITY",
          -4: "NWC_ERR_FORMAT", -5: "NWC_ERR_HIP", -6: "NWC_ERR_UNSUPPORTED"}

EXPORTS = ("nwc_version", "nwc_status_string", "nwc_encode_bound", "nwc_encode", "nwc_encode_ex", "nwc_blob_info", "nwc_blob_check",
           "nwc_workspace_size", "nwc_matvec", "nwc_matvec_noalloc", "nwc_matvec_group", "nwc_matvec_batch", "nwc_dequant", "nwc_gather", "nwc_stream_read",
           "nwc_bf16_gemv", "nwc_bf16_gemv_group")


class NWCError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {msg}")
        self.status = status


class NWCInfo(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("elem", ctypes.c_int32),
                ("cols_per_lane", ctypes.c_int32), ("rows_per_wave", ctypes.c_int32),
                ("waves_per_group", ctypes.c_int32), ("n_spans", ctypes.c_int32), ("n_items", ctypes.c_int32),
                ("max_rows", ctypes.c_int32), ("coder", ctypes.c_int32),
                ("coded_bits", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64),
                ("code_bytes", ctypes.c_uint64), ("mant_bytes", ctypes.c_uint64),
                ("table_bytes", ctypes.c_uint64), ("rank_to_sym", ctypes.c_uint8 * 128)]


class MatvecDesc(ctypes.Structure):
    """One member of nwc_matvec_group: the arguments of nwc_matvec without the workspace."""
    _fields_ = [("header", ctypes.c_void_p), ("d_blob", ctypes.c_void_p), ("d_x", ctypes.c_void_p),
                ("d_scale", ctypes.c_void_p), ("d_y", ctypes.c_void_p)]


class GemvDesc(ctypes.Structure):
    """One member of nwc_bf16_gemv_group: the arguments of nwc_bf16_gemv."""
    _fields_ = [("d_w", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("ldw", ctypes.c_int64),
                ("d_x", ctypes.c_void_p), ("d_y", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libnwc.so not built ({LIB_PATH}); run `python -m decode_matvec_amd.build`")
    # PyTorch ships its own HIP runtime (soname libamdhip64.so.7, which also
    # satisfies this library) but asks for it by the unversioned name.  Loaded
    # first, this library would bind /opt/rocm's runtime and PyTorch would
    # then load its own beside it: two HIP runtimes in one process, and the
    # library's finds no device.  Importing torch first leaves one runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    sig = {
        "nwc_version": ([], ci),
        "nwc_status_string": ([ci], ctypes.c_char_p),
        "nwc_encode_bound": ([i64, i64, ci, ci, ci, ctypes.POINTER(i64)], ci),
        "nwc_encode": ([vp, i64, i64, i64, ci, ci, ci, vp, i64, ctypes.POINTER(i64)], ci),
        "nwc_encode_ex": ([vp, i64, i64, i64, ci, ci, ci, ci, vp, i64, ctypes.POINTER(i64)], ci),
        "nwc_blob_info": ([vp, i64, ctypes.POINTER(NWCInfo)], ci),
        "nwc_blob_check": ([vp, i64], ci),
        "nwc_workspace_size": ([vp, ctypes.POINTER(i64)], ci),
        "nwc_matvec": ([vp, vp, vp, vp, vp, vp, i64, vp], ci),
        "nwc_matvec_noalloc": ([vp, vp, vp, vp, vp, vp], ci),
        "nwc_matvec_group": ([ctypes.POINTER(MatvecDesc), ci, vp], ci),
        "nwc_matvec_batch": ([vp, vp, vp, i64, i64, vp, vp, i64, vp, i64, vp], ci),
        "nwc_dequant": ([vp, vp, vp, i64, vp], ci),
        "nwc_gather": ([vp, vp, vp, i64, vp, vp], ci),
        "nwc_stream_read": ([vp, i64, vp, vp], ci),
        "nwc_bf16_gemv": ([vp, i64, i64, i64, vp, vp, vp], ci),
        "nwc_bf16_gemv_group": ([ctypes.POINTER(GemvDesc), ci, vp], ci),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


lib = _load()


def _check(fn: str, st: int):
    if st != 0:
        raise NWCError(fn, st, lib.nwc_status_string(st).decode())


def version() -> int:
    return lib.nwc_version()


def status_string(st: int) -> str:
    return lib.nwc_status_string(st).decode()


def _host_ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def encode_bound(n: int, k: int, elem: int = NWC_BF16, cols_per_lane: int = 0, rows_per_wave: int = 0) -> int:
    out = ctypes.c_int64()
    _check("nwc_encode_bound", lib.nwc_encode_bound(n, k, elem, cols_per_lane, rows_per_wave, ctypes.byref(out)))
    return out.value


def encode(w: np.ndarray, elem: int = NWC_BF16, cols_per_lane: int = 0, rows_per_wave: int = 0,
           coder: int = NWC_CODER_UNARY) -> np.ndarray:
    """Encode a host matrix (uint16 BF16 patterns or uint8 fp8 bytes) -> uint8 blob.

    cols_per_lane / rows_per_wave: 0 lets the library choose the work-item geometry.
    coder: NWC_CODER_UNARY (the pages' code) or NWC_CODER_HUFFMAN (fp8 bytes, length-limited Huffman)."""
    want = np.uint16 if elem == NWC_BF16 else np.uint8
    if w.dtype != want or w.ndim != 2:
        raise TypeError(f"expected a 2-D {np.dtype(want).name} array, got {w.dtype} {w.shape}")
    if w.strides[1] != w.itemsize:
        w = np.ascontiguousarray(w)
    n, k = w.shape
    ld = w.strides[0] // w.itemsize
    cap = encode_bound(n, k, elem, cols_per_lane, rows_per_wave)
    blob = np.empty(cap, dtype=np.uint8)
    size = ctypes.c_int64()
    _check("nwc_encode_ex", lib.nwc_encode_ex(_host_ptr(w), n, k, ld, elem, coder, cols_per_lane, rows_per_wave,
                                              _host_ptr(blob), cap, ctypes.byref(size)))
    return blob[:size.value].copy()


def blob_info(blob: np.ndarray) -> dict:
    info = NWCInfo()
    _check("nwc_blob_info", lib.nwc_blob_info(_host_ptr(blob), blob.nbytes, ctypes.byref(info)))
    d = {f: getattr(info, f) for f, _ in NWCInfo._fields_ if f != "rank_to_sym"}
    d["rank_to_sym"] = list(info.rank_to_sym)
    return d


def blob_check(blob: np.ndarray) -> None:
    """Full host-side validation of a blob (header, rank and decode tables, item table); raises NWCError."""
    _check("nwc_blob_check", lib.nwc_blob_check(_host_ptr(blob), blob.nbytes))


def workspace_size(header: np.ndarray) -> int:
    out = ctypes.c_int64()
    _check("nwc_workspace_size", lib.nwc_workspace_size(_host_ptr(header), ctypes.byref(out)))
    return out.value


def _dev(t):
    return 0 if t is None else t.data_ptr()


def _need(fn: str, what: str, t, min_elems: int, elem_size: int, floating=None):
    """Host-side check of a device tensor argument before its pointer reaches the library: a CUDA/HIP tensor,
    contiguous, of the element size the entry point reads or writes, holding at least ``min_elems`` elements.
    ``floating``: True requires a floating dtype (fp32 outputs, scales), False an integer one (ids)."""
    if t is None:
        raise ValueError(f"{fn}: {what} is required")
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{fn}: {what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{fn}: {what} must be contiguous")
    if t.element_size() != elem_size:
        raise ValueError(f"{fn}: {what} needs {elem_size}-byte elements, got {t.dtype}")
    if floating is not None and t.dtype.is_floating_point != floating:
        raise ValueError(f"{fn}: {what} has dtype {t.dtype}")
    if t.numel() < min_elems:
        raise ValueError(f"{fn}: {what} holds {t.numel()} elements, needs {min_elems}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _shape(header: np.ndarray):
    """(n, k, elem) read from the host header copy (validated by the library on every call)."""
    h = np.frombuffer(np.ascontiguousarray(header[:32]).tobytes(), dtype=np.uint8)
    elem = int(h[8:12].view(np.uint32)[0])
    n, k = (int(v) for v in h[16:32].view(np.int64))
    return n, k, elem


def matvec(header: np.ndarray, d_blob, x, y, ws=None, scale=None, stream=None) -> None:
    """y[n] (fp32) = W x (times scale for fp8) on the GPU; all device arguments are torch tensors."""
    n, k, elem = _shape(header)
    _need("nwc_matvec", "x", x, k, 2)
    _need("nwc_matvec", "y", y, n, 4, floating=True)
    if elem == NWC_FP8_E4M3:
        _need("nwc_matvec", "scale", scale, n, 4, floating=True)
    _check("nwc_matvec", lib.nwc_matvec(_host_ptr(header), _dev(d_blob), _dev(x), _dev(scale), _dev(y), _dev(ws),
                                        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 4 << 20


def matvec_noalloc(header: np.ndarray, d_blob, x, y, scale=None, stream=None) -> None:
    """nwc_matvec without a workspace: split-row partials live in the library's static per-GPU scratch."""
    n, k, elem = _shape(header)
    _need("nwc_matvec_noalloc", "x", x, k, 2)
    _need("nwc_matvec_noalloc", "y", y, n, 4, floating=True)
    if elem == NWC_FP8_E4M3:
        _need("nwc_matvec_noalloc", "scale", scale, n, 4, floating=True)
    _check("nwc_matvec_noalloc", lib.nwc_matvec_noalloc(_host_ptr(header), _dev(d_blob), _dev(x), _dev(scale),
                                                        _dev(y), _stream(stream)))


def matvec_group(mats, xs, ys, scales=None, stream=None) -> None:
    """y_m = W_m x_m for every DeviceMatrix in ``mats`` in one launch per work-item shape (nwc_matvec_group).

    xs / ys / scales: one device tensor per matrix (scales: None, or a list with fp32 scales for fp8 members)."""
    count = len(mats)
    if len(xs) != count or len(ys) != count or (scales is not None and len(scales) != count):
        raise ValueError("nwc_matvec_group: one activation, output (and scale) per matrix")
    if count > GROUP_MAX:
        raise ValueError(f"nwc_matvec_group: at most {GROUP_MAX} matrices")
    descs = (MatvecDesc * max(1, count))()
    for i, dm in enumerate(mats):
        sc = None if scales is None else scales[i]
        _need("nwc_matvec_group", f"x[{i}]", xs[i], dm.k, 2)
        _need("nwc_matvec_group", f"y[{i}]", ys[i], dm.n, 4, floating=True)
        if dm.elem == NWC_FP8_E4M3:
            _need("nwc_matvec_group", f"scale[{i}]", sc, dm.n, 4, floating=True)
        descs[i] = MatvecDesc(_host_ptr(dm.header), _dev(dm.d_blob), _dev(xs[i]), _dev(sc), _dev(ys[i]))
    _check("nwc_matvec_group", lib.nwc_matvec_group(descs, count, _stream(stream)))


def matvec_batch(header: np.ndarray, d_blob, x, y, ws=None, scale=None, stream=None) -> None:
    """y[b] (fp32 rows) = W x[b] for the rows of x (batch x ldx BF16 patterns) into y (batch x ldy fp32)."""
    n, k, elem = _shape(header)
    if x.dim() != 2 or y.dim() != 2:
        raise ValueError("nwc_matvec_batch: x and y must be 2-D (rows x elements)")
    batch = x.shape[0]
    if y.shape[0] != batch:
        raise ValueError("x and y need the same number of rows")
    if x.shape[1] < k or y.shape[1] < n:
        raise ValueError(f"nwc_matvec_batch: rows of x need >= {k} elements and rows of y >= {n}")
    _need("nwc_matvec_batch", "x", x, batch * x.shape[1], 2)
    _need("nwc_matvec_batch", "y", y, batch * y.shape[1], 4, floating=True)
    if elem == NWC_FP8_E4M3:
        _need("nwc_matvec_batch", "scale", scale, n, 4, floating=True)
    _check("nwc_matvec_batch", lib.nwc_matvec_batch(_host_ptr(header), _dev(d_blob), _dev(x), x.stride(0), batch,
                                                    _dev(scale), _dev(y), y.stride(0), _dev(ws),
                                                    0 if ws is None else ws.numel() * ws.element_size(),
                                                    _stream(stream)))


def dequant(header: np.ndarray, d_blob, out, ld: int, stream=None) -> None:
    """Rows of the matrix into out (row i at element i*ld): BF16 patterns, or fp8 bytes."""
    n, k, elem = _shape(header)
    if ld < k:
        raise ValueError(f"nwc_dequant: ld {ld} < k {k}")
    _need("nwc_dequant", "out", out, (n - 1) * ld + k, 2 if elem == NWC_BF16 else 1)
    _check("nwc_dequant", lib.nwc_dequant(_host_ptr(header), _dev(d_blob), _dev(out), ld, _stream(stream)))


def stream_read(buf, sink, nbytes=None, stream=None) -> None:
    """Plain streaming read of a device tensor (measurement reference); sink: one int32 on the device."""
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check("nwc_stream_read", lib.nwc_stream_read(_dev(buf), n, _dev(sink), _stream(stream)))


def bf16_gemv(w, x, y, stream=None, k=None) -> None:
    """Plain BF16 GEMV y = W x (the uncompressed measurement baseline): w int16/bfloat16 [n, ldw] device
    (row pitch w.stride(0)), x [k] device, y fp32 [n] device.  k defaults to w.shape[1]."""
    if w.dim() != 2:
        raise ValueError("nwc_bf16_gemv: w must be 2-D")
    n, ldw = w.shape
    k = ldw if k is None else int(k)
    if k > ldw:
        raise ValueError(f"nwc_bf16_gemv: k {k} > columns of w {ldw}")
    if w.element_size() != 2 or not w.is_cuda or w.stride(1) != 1:
        raise ValueError("nwc_bf16_gemv: w must be a device tensor of 2-byte elements with unit column stride")
    _need("nwc_bf16_gemv", "x", x, k, 2)
    _need("nwc_bf16_gemv", "y", y, n, 4, floating=True)
    _check("nwc_bf16_gemv", lib.nwc_bf16_gemv(_dev(w), n, k, w.stride(0), _dev(x), _dev(y),
                                              _stream(stream)))


def bf16_gemv_group(ws, xs, ys, stream=None) -> None:
    """Several plain BF16 GEMVs y_m = W_m x_m in one launch (measurement baseline); w: [n, ldw] device tensors."""
    count = len(ws)
    if len(xs) != count or len(ys) != count or count > GROUP_MAX:
        raise ValueError("nwc_bf16_gemv_group: one activation and output per matrix, at most GROUP_MAX matrices")
    descs = (GemvDesc * max(1, count))()
    for i, w in enumerate(ws):
        if w.dim() != 2 or w.element_size() != 2 or not w.is_cuda or w.stride(1) != 1:
            raise ValueError("nwc_bf16_gemv_group: w must be a 2-D device tensor of 2-byte elements")
        n, k = w.shape
        _need("nwc_bf16_gemv_group", f"x[{i}]", xs[i], k, 2)
        _need("nwc_bf16_gemv_group", f"y[{i}]", ys[i], n, 4, floating=True)
        descs[i] = GemvDesc(_dev(w), n, k, w.stride(0), _dev(xs[i]), _dev(ys[i]))
    _check("nwc_bf16_gemv_group", lib.nwc_bf16_gemv_group(descs, count, _stream(stream)))


def gather(header: np.ndarray, d_blob, ids, out, stream=None) -> None:
    """Rows ids[t] of the matrix into out[t] (k elements each); ids outside [0, n) give zero rows."""
    n, k, elem = _shape(header)
    _need("nwc_gather", "ids", ids, 0, 8, floating=False)
    _need("nwc_gather", "out", out, ids.numel() * k, 2 if elem == NWC_BF16 else 1)
    _check("nwc_gather", lib.nwc_gather(_host_ptr(header), _dev(d_blob), _dev(ids), ids.numel(), _dev(out),
                                        _stream(stream)))


class DeviceMatrix:
    """A compressed matrix resident on the GPU: host header copy + device blob + workspace.

    Holds buffers only; every computation is a call into libnwc."""

    def __init__(self, blob: np.ndarray, device="cuda"):
        import torch
        self.info = blob_info(blob)
        self.header = np.ascontiguousarray(blob[:HEADER_BYTES]).copy()
        self.d_blob = torch.from_numpy(blob).to(device)
        wsb = workspace_size(self.header)
        self.ws = torch.empty(wsb // 4, dtype=torch.int32, device=device) if wsb else None
        self.n, self.k = self.info["n"], self.info["k"]
        self.elem = self.info["elem"]
        self.nbytes = int(blob.nbytes)

    def matvec(self, x, y, scale=None, stream=None):
        matvec(self.header, self.d_blob, x, y, self.ws, scale, stream)

    def matvec_batch(self, x, y, scale=None, stream=None):
        matvec_batch(self.header, self.d_blob, x, y, self.ws, scale, stream)

    def dequant(self, out, ld=None, stream=None):
        dequant(self.header, self.d_blob, out, self.k if ld is None else ld, stream)

    def gather(self, ids, out, stream=None):
        gather(self.header, self.d_blob, ids, out, stream)
