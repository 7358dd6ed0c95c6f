"""Test-side reader of the library's blob layout (slow, CPU, small matrices).

Reads the header and the per-item lane streams exactly as the stream layout
is documented in decode_matvec_amd/csrc/nwc_format.h, and decodes them with
the oracle's one-code parser.  This checks the host encoder's layout on the
CPU, without a GPU; it is test code, not part of the product.
"""
import numpy as np

import oracle as O

HDR = np.dtype([("magic", "<u4"), ("version", "<u4"), ("elem", "<u4"), ("header_bytes", "<u4"),
                ("n", "<i8"), ("k", "<i8"), ("cols_per_item", "<u4"), ("n_rowblocks", "<u4"),
                ("n_kspans", "<u4"), ("n_items", "<u4"), ("max_rows", "<u4"), ("escape_r", "<u4"),
                ("last_cols", "<u4"), ("k_pad", "<u4"), ("coded_bits", "<u8"), ("off_lut", "<u8"),
                ("off_items", "<u8"), ("off_mant", "<u8"), ("off_code", "<u8"), ("total_bytes", "<u8"),
                ("code_bytes", "<u8"), ("mant_bytes", "<u8"), ("rank_to_sym", "u1", (128,))])
assert HDR.itemsize == 256


def header(blob: np.ndarray) -> dict:
    h = np.frombuffer(blob[:256].tobytes(), dtype=HDR)[0]
    return {name: (h[name] if name == "rank_to_sym" else int(h[name])) for name in HDR.names}


def lane_bits(blob, h, item, lane):
    off, rows = np.frombuffer(blob[h["off_items"] + 8 * item: h["off_items"] + 8 * item + 8].tobytes(), "<u4")
    base = h["off_code"] + int(off)
    words = np.frombuffer(blob[base: base + int(rows) * 256].tobytes(), "<u4").reshape(int(rows), 64)[:, lane]
    return np.unpackbits(words.astype("<u4").view(np.uint8), bitorder="little")


def decode_blob(blob: np.ndarray) -> np.ndarray:
    """Whole matrix from a library blob (uint16 BF16 patterns or uint8 fp8 bytes)."""
    h = header(blob)
    n, k, C = h["n"], h["k"], h["cols_per_item"]
    fp8 = h["elem"] == 1
    r2s = np.array(h["rank_to_sym"][: 16 if fp8 else 128], dtype=np.int64)
    out = np.zeros((n, k), dtype=np.uint8 if fp8 else np.uint16)
    for rb in range(h["n_rowblocks"]):
        for ks in range(h["n_kspans"]):
            item = rb * h["n_kspans"] + ks
            c0 = ks * C
            nc = h["last_cols"] if ks == h["n_kspans"] - 1 else C
            mbase = h["off_mant"] + rb * 64 * h["k_pad"] + 64 * c0
            for L in range(64):
                row = rb * 64 + L
                if row >= n:
                    break
                bits = list(lane_bits(blob, h, item, L)) + [0] * 32
                assert bits[0] == 0 and bits[1] == 0
                pos = 2
                for c in range(nc):
                    if fp8:
                        r = 0
                        while r < 8 and bits[pos + r] == 1:
                            r += 1
                        if r < 8:
                            s = bits[pos + r + 1]
                            M = bits[pos + r + 2] | bits[pos + r + 3] << 1 | bits[pos + r + 4] << 2
                            E = int(r2s[r])
                            pos += r + 5
                        else:
                            s = bits[pos + 8]
                            E = sum(bits[pos + 9 + i] << i for i in range(4))
                            M = sum(bits[pos + 13 + i] << i for i in range(3))
                            pos += 16
                        out[row, c0 + c] = (s << 7) | (E << 3) | M
                    else:
                        s, e, pos = O.parse_one_bf16(bits, pos, r2s)
                        m = blob[mbase + ((c >> 4) * 64 + L) * 16 + (c & 15)]
                        out[row, c0 + c] = (s << 15) | (e << 8) | int(m)
    return out


def lut(blob: np.ndarray) -> np.ndarray:
    h = header(blob)
    return np.frombuffer(blob[h["off_lut"]: h["off_lut"] + 16384].tobytes(), "<u4")
