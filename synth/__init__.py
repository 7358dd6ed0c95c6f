"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module only draws numbers and rounds them to the storage formats the
workloads are defined in (BF16, fp8 e4m3fn).  It contains none of the codec's
arithmetic: no byte split, no ranking, no codewords, no matrix-vector product.
Both the CPU oracle (``oracle/``) and the GPU path consume its outputs, and
neither depends on the other.

Recipes (all seeds fixed; see ``configs``):

* weights: fp32 standard normal draws times an fp32 standard deviation, rounded
  to BF16 with round-to-nearest-even; activations likewise with sigma 1.
* small matrices (the 1024 x 1024 matrix, the odd shapes) draw the whole
  matrix in row-major order from numpy's PCG64 ``default_rng(seed)``;
  the workload matrices of the decoder layer sets and the embedding tables
  draw in blocks of 256 rows, block b from
  ``Generator(PCG64(SeedSequence(seed, spawn_key=(b,))))`` (the b-th child of
  ``SeedSequence(seed).spawn``), so that the blocks of billions of draws can be
  made on several host threads and every consumer -- the CPU oracle tests, the
  GPU tests, the benchmark -- sees the same matrices.  Which recipe a matrix
  uses is part of its workload definition (``synth.configs``).
* heavy-tailed weights: 0.02 times a Student-t draw with 3 degrees of freedom.
* rare values are injected at seeded positions to exercise the escape code.
* fp8 weights: symmetric per-output-channel absmax scaling to the e4m3fn range,
  then round-to-nearest-even (torch's float8_e4m3fn cast).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_from_f32", "f32_from_bf16", "normal_bf16", "student_t_bf16", "inject_rare",
    "all_patterns_bf16", "all_bytes_fp8", "fp8_quantize", "token_ids", "activation_bf16",
    "blocked_normal_bf16", "BLOCK_ROWS", "odd_shape_matrix",
]


def bf16_from_f32(a) -> np.ndarray:
    """Round fp32 values to BF16 bit patterns (uint16), nearest-even; NaNs stay NaN."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def f32_from_bf16(u16) -> np.ndarray:
    """Exact fp32 value of BF16 bit patterns."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: int, shape, sigma: float) -> np.ndarray:
    """BF16 bits of fp32 N(0, sigma) draws (sigma is the standard deviation)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(shape, dtype=np.float32)
    z *= np.float32(sigma)
    return bf16_from_f32(z)


def activation_bf16(seed: int, k: int) -> np.ndarray:
    return normal_bf16(seed, (k,), 1.0)


def student_t_bf16(seed: int, shape, scale: float = 0.02, df: float = 3.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    t = rng.standard_t(df, size=shape).astype(np.float32)
    t *= np.float32(scale)
    return bf16_from_f32(t)


# Rare BF16 patterns cycled through at injected positions: tiny and huge
# magnitudes, both zeros, and subnormals.  Inf/NaN are excluded here because the
# matvec tolerance needs a finite sum |w*x|; they appear in all_patterns_bf16.
_RARE = np.concatenate([
    bf16_from_f32(np.array([1e-30, -1e-30, 1e4, -1e4], np.float32)),
    np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F], np.uint16),
])


def inject_rare(u16: np.ndarray, seed: int, frac: float = 1e-3, minimum: int = 8) -> np.ndarray:
    """Copy of ``u16`` with rare values written at seeded positions.

    At least ``minimum`` positions (or ``frac`` of the elements, if more) are
    overwritten, cycling through fixed rare patterns plus random-mantissa
    subnormals."""
    out = np.array(u16, dtype=np.uint16, copy=True)
    flat = out.reshape(-1)
    n = flat.size
    cnt = min(n, max(minimum, int(round(frac * n))))
    rng = np.random.default_rng(seed)
    pos = rng.choice(n, size=cnt, replace=False)
    vals = np.empty(cnt, np.uint16)
    for i in range(cnt):
        j = i % (len(_RARE) + 1)
        if j < len(_RARE):
            vals[i] = _RARE[j]
        else:  # subnormal with a random nonzero mantissa and random sign
            vals[i] = np.uint16(int(rng.integers(1, 128)) | (int(rng.integers(0, 2)) << 15))
    flat[pos] = vals
    return out


def all_patterns_bf16() -> np.ndarray:
    """256 x 256 matrix holding every BF16 bit pattern once: u[i][j] = i<<8 | j."""
    i = np.arange(256, dtype=np.uint16)[:, None]
    j = np.arange(256, dtype=np.uint16)[None, :]
    return (i << 8) | j


def all_bytes_fp8(rows: int = 4) -> np.ndarray:
    """``rows`` x 256 matrix of fp8 bytes, each row holding all 256 patterns."""
    return np.tile(np.arange(256, dtype=np.uint8), (rows, 1))


def fp8_quantize(w_u16: np.ndarray):
    """Weight-only fp8 e4m3fn quantization with a symmetric per-row scale.

    scale_i = max_j |w_ij| / 448 in fp32 (1 if the row is all zero);
    q_ij = e4m3fn_rne(clamp(w_ij / scale_i, -448, 448)).
    Returns (q bytes uint8 [N, K], scale float32 [N])."""
    import torch
    w = f32_from_bf16(w_u16).reshape(w_u16.shape)
    amax = np.abs(w).max(axis=1).astype(np.float32)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale[scale == 0] = np.float32(1.0)
    v = np.clip(w / scale[:, None], np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    q = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.ascontiguousarray(q), scale


def token_ids(seed: int, vocab: int, n: int) -> np.ndarray:
    """``n`` uniform token ids in [0, vocab), drawn with replacement."""
    return np.random.default_rng(seed).integers(0, vocab, size=n, dtype=np.int64)


BLOCK_ROWS = 256


def blocked_normal_bf16(seed: int, shape, sigma: float, threads: int | None = None) -> np.ndarray:
    """BF16 bits of fp32 N(0, sigma) draws, rows drawn in blocks of BLOCK_ROWS.

    Block b (rows [256 b, 256 b + 256)) is drawn row-major from
    ``Generator(PCG64(SeedSequence(seed, spawn_key=(b,))))``: fp32 standard
    normal draws times fp32(sigma), then round-to-nearest-even to BF16.  The
    result does not depend on ``threads``."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    n, k = shape
    out = np.empty((n, k), np.uint16)
    sig = np.float32(sigma)

    def one(b):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(int(seed), spawn_key=(b,))))
        r0, r1 = b * BLOCK_ROWS, min(n, (b + 1) * BLOCK_ROWS)
        z = g.standard_normal((r1 - r0, k), dtype=np.float32)
        z *= sig
        out[r0:r1] = bf16_from_f32(z)

    nb = (n + BLOCK_ROWS - 1) // BLOCK_ROWS
    with ThreadPoolExecutor(max(1, min(nb, threads or os.cpu_count() or 1))) as ex:
        list(ex.map(one, range(nb)))
    return out


def odd_shape_matrix(idx: int, kind: str):
    """The odd-shape workload's matrix ``idx`` of kind "normal" (N(0, 0.02)) or
    "t3" (0.02 t3), with rare values injected; returns (w, x, seed).

    Seed 300000 + 2 idx (+1 for t3); rare positions from seed + 50; the
    activation from seed + 60."""
    from . import configs as C
    n, k = C.ODD_SHAPES[idx]
    seed = C.odd_seed(2 * idx + (kind == "t3"))
    w = normal_bf16(seed, (n, k), 0.02) if kind == "normal" else student_t_bf16(seed, (n, k))
    return inject_rare(w, seed + 50), activation_bf16(seed + 60, k), seed
