"""Test-side reader of the library's blob layout (slow, CPU, small matrices).

Reads the header and the per-item lane streams exactly as the stream layout
is documented in decode_matvec_amd/csrc/nwc_format.h, and decodes them with
the oracle's one-code parser.  This checks the host encoder's layout on the
CPU, without a GPU; it is test code, not part of the product.
"""
import numpy as np

import oracle as O

HDR = np.dtype([("magic", "<u4"), ("version", "<u4"), ("elem", "<u4"), ("header_bytes", "<u4"),
                ("n", "<i8"), ("k", "<i8"), ("cols_per_lane", "<u4"), ("rows_per_wave", "<u4"),
                ("waves_per_group", "<u4"), ("n_spans", "<u4"), ("n_rowgroups", "<u4"), ("n_items", "<u4"),
                ("max_rows", "<u4"), ("escape_r", "<u4"), ("coded_bits", "<u8"), ("off_lut", "<u8"),
                ("off_items", "<u8"), ("off_mant", "<u8"), ("off_code", "<u8"), ("total_bytes", "<u8"),
                ("code_bytes", "<u8"), ("mant_bytes", "<u8"), ("rank_to_sym", "u1", (128,))])
assert HDR.itemsize == 256


def header(blob: np.ndarray) -> dict:
    h = np.frombuffer(blob[:256].tobytes(), dtype=HDR)[0]
    return {name: (h[name] if name == "rank_to_sym" else int(h[name])) for name in HDR.names}


def lane_place(h, item, lane):
    """(row, first column) of lane `lane` of work item `item`."""
    R, W, sp = h["rows_per_wave"], h["waves_per_group"], h["n_spans"]
    S, C = 64 // R, h["cols_per_lane"]
    group, wave = divmod(item, W)
    rg, span = divmod(group, sp)
    q = (span * W + wave) * S + lane % S
    return rg * R + lane // S, q * C


def lane_bits(blob, h, item, lane):
    off, rows = np.frombuffer(blob[h["off_items"] + 8 * item: h["off_items"] + 8 * item + 8].tobytes(), "<u4")
    base = h["off_code"] + int(off)
    words = np.frombuffer(blob[base: base + int(rows) * 256].tobytes(), "<u4").reshape(int(rows), 64)[:, lane]
    return np.unpackbits(words.astype("<u4").view(np.uint8), bitorder="little")


def mant_byte(blob, h, item, lane, c):
    return blob[h["off_mant"] + item * 64 * h["cols_per_lane"] + ((c >> 4) * 64 + lane) * 16 + (c & 15)]


def _parse_fp8(bits, pos, r2s):
    r = 0
    while r < 8 and bits[pos + r] == 1:
        r += 1
    if r < 8:
        s = bits[pos + r + 1]
        M = bits[pos + r + 2] | bits[pos + r + 3] << 1 | bits[pos + r + 4] << 2
        return (s << 7) | (int(r2s[r]) << 3) | M, pos + r + 5
    s = bits[pos + 8]
    E = sum(bits[pos + 9 + i] << i for i in range(4))
    M = sum(bits[pos + 13 + i] << i for i in range(3))
    return (s << 7) | (E << 3) | M, pos + 16


def huffman_lengths(h) -> list:
    """Codeword length of each fp8 byte of a Huffman-variant blob (nibbles of the rank_to_sym field)."""
    r = h["rank_to_sym"]
    return [int(r[b // 2]) >> (4 * (b & 1)) & 15 for b in range(256)]


def _huffman_parser(h):
    codes = O.canonical_codes(huffman_lengths(h))
    by_bits = {tuple(O.codeword_huffman(c, l)): s for s, (c, l) in codes.items()}

    def parse(bits, pos):
        for l in range(1, O.HUFF_MAX_LEN + 1):
            s = by_bits.get(tuple(bits[pos:pos + l]))
            if s is not None:
                return s, pos + l
        raise AssertionError("no codeword")
    return parse


def decode_blob(blob: np.ndarray) -> np.ndarray:
    """Whole matrix from a library blob (uint16 BF16 patterns or uint8 fp8 bytes).

    Also asserts the filler convention: every lane stream starts with two zero
    bits, and stream bits past a lane's real columns (after the Huffman
    variant's filler codewords of byte 0x00), and mantissa bytes of filler
    columns, are zero."""
    h = header(blob)
    n, k, C = h["n"], h["k"], h["cols_per_lane"]
    fp8 = h["elem"] == 1
    huff = fp8 and h["escape_r"] == 0
    parse_h = _huffman_parser(h) if huff else None
    r2s = np.array(h["rank_to_sym"][: 16 if fp8 else 128], dtype=np.int64)
    out = np.zeros((n, k), dtype=np.uint8 if fp8 else np.uint16)
    seen = np.zeros((n, k), dtype=bool)
    for item in range(h["n_items"]):
        for L in range(64):
            row, c0 = lane_place(h, item, L)
            bits = lane_bits(blob, h, item, L)
            assert bits[0] == 0 and bits[1] == 0
            real = max(0, min(k - c0, C)) if row < n else 0
            pos = 2
            padded = list(bits) + [0] * 32
            for c in range(real):
                if huff:
                    b, pos = parse_h(padded, pos)
                    out[row, c0 + c] = b
                elif fp8:
                    b, pos = _parse_fp8(padded, pos, r2s)
                    out[row, c0 + c] = b
                else:
                    s, e, pos = O.parse_one_bf16(padded, pos, r2s)
                    out[row, c0 + c] = (s << 15) | (e << 8) | int(mant_byte(blob, h, item, L, c))
                seen[row, c0 + c] = True
            if huff:   # fillers: byte 0x00's codeword up to C codes per lane
                for c in range(real, C):
                    b, pos = parse_h(padded, pos)
                    assert b == 0, (item, L, c)
            assert not np.any(bits[pos:]), (item, L)
            if not fp8:
                for c in range(real, C):
                    assert mant_byte(blob, h, item, L, c) == 0, (item, L, c)
    assert seen.all()
    return out


def lut(blob: np.ndarray) -> np.ndarray:
    h = header(blob)
    return np.frombuffer(blob[h["off_lut"]: h["off_lut"] + 16384].tobytes(), "<u4")
