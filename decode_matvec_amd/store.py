"""Files of encoded matrices: one safetensors file, every blob stored whole.

NWC project page (PyPI, usage after "Install"): a compressed checkpoint is
saved once and later loaded straight to the GPU without the BF16 originals.
Here a blob is self-describing (header, decode table, item table, planes), so
the file holds each blob as a uint8 tensor under the caller's name, next to any
plain arrays the caller adds (fp8 row scales, norm weights).  The file's
metadata marks the format and names the blobs (each blob header carries its
own format version, which the check below compares with the library's).

load() runs the library's full check (nwc_blob_check: header, rank and decode
tables, item table) on every blob before returning it: the device kernels trust
a blob's item table, whose offsets bound their memory accesses, so a damaged
or foreign file is rejected on the host.  Host code only.
"""
from __future__ import annotations

import numpy as np
from safetensors.numpy import load_file, save_file

from . import nwc

FORMAT = "nwc-blobs"


def save(path: str, blobs: dict[str, np.ndarray], arrays: dict[str, np.ndarray] | None = None) -> None:
    """Writes `blobs` (name -> uint8 blob from nwc.encode) and `arrays` (name -> any numpy array) to `path`.

    Every blob is checked first (nwc_blob_check); names must be distinct across both dicts."""
    arrays = arrays or {}
    clash = set(blobs) & set(arrays)
    if any("," in n for n in blobs):
        raise ValueError("blob names may not contain ','")
    if clash:
        raise ValueError(f"names used for both a blob and an array: {sorted(clash)}")
    tensors = {}
    for name, b in blobs.items():
        b = np.ascontiguousarray(b)
        if b.dtype != np.uint8 or b.ndim != 1:
            raise ValueError(f"blob {name!r}: expected a 1-D uint8 array, got {b.dtype} {b.shape}")
        nwc.blob_check(b)
        tensors[name] = b
    for name, a in arrays.items():
        tensors[name] = np.ascontiguousarray(a)
    meta = {"format": FORMAT, "blobs": ",".join(sorted(blobs))}
    save_file(tensors, path, metadata=meta)


def load(path: str) -> tuple[dict[str, np.ndarray], dict[str, np.ndarray]]:
    """Reads a file written by save(): (blobs, arrays), every blob fully checked (raises nwc.NWCError)."""
    from safetensors import safe_open

    with safe_open(path, framework="numpy") as f:
        meta = f.metadata() or {}
    if meta.get("format") != FORMAT:
        raise ValueError(f"{path}: not an NWC blob file (format {meta.get('format')!r})")
    names = set(filter(None, meta.get("blobs", "").split(",")))
    tensors = load_file(path)
    missing = names - set(tensors)
    if missing:
        raise ValueError(f"{path}: blobs listed but absent: {sorted(missing)}")
    blobs, arrays = {}, {}
    for name, t in tensors.items():
        if name in names:
            if t.dtype != np.uint8 or t.ndim != 1:
                raise ValueError(f"{path}: blob {name!r} is {t.dtype} {t.shape}")
            nwc.blob_check(t)
            blobs[name] = t
        else:
            arrays[name] = t
    return blobs, arrays
