"""Several tokens at once (prefill): dequantize, then a library GEMM.

NWC project page ("How it works", the dequantization bullet): for batch > 1
the blob is dequantized into a temporary BF16 buffer and the product runs in
the vendor BLAS; the pages add that this saves memory, not time.  Here the
dequantization is nwc_dequant (bit-exact) and the GEMM is
torch.nn.functional.linear (hipBLASLt / rocBLAS on ROCm), so for a BF16 blob
the result equals F.linear on the original weights bit for bit.  An fp8 blob
dequantizes to its e4m3 bytes, which widen exactly to BF16; the row scale then
multiplies the fp32 GEMM output (model card: scale after the row sum).

For one to four tokens nwc_matvec / nwc_matvec_batch read the compressed bytes
only and are faster; this path is for longer batches, where the GEMM is
compute-bound and a BF16 copy of one matrix at a time is affordable.
"""
from __future__ import annotations

from . import nwc


def scratch_for(dm: "nwc.DeviceMatrix"):
    """A dequantization buffer for `dm` (reusable across matrices of the same or smaller size and element type)."""
    import torch
    dtype = torch.int16 if dm.elem == nwc.NWC_BF16 else torch.uint8
    return torch.empty((dm.n, dm.k), dtype=dtype, device=dm.d_blob.device)


def prefill(dm: "nwc.DeviceMatrix", x, scale=None, scratch=None):
    """Y = X · Wᵀ for X [T, K] bfloat16 on the blob's device → Y [T, N] bfloat16.

    scale: fp32 [N] row scales, required for an fp8 blob and refused for a BF16 one.
    scratch: optional buffer from scratch_for() (int16 [N, K] for BF16, uint8 [N, K] for fp8; a larger
    one is used through its first N·K elements); allocated per call when None.
    Runs on torch's current stream (the dequantization and the GEMM both)."""
    import torch
    import torch.nn.functional as F

    if x.dim() != 2 or x.shape[1] != dm.k or x.dtype != torch.bfloat16:
        raise ValueError(f"x must be bfloat16 [T, {dm.k}], got {x.dtype} {tuple(x.shape)}")
    fp8 = dm.elem == nwc.NWC_FP8_E4M3
    if fp8 != (scale is not None):
        raise ValueError("an fp8 blob needs its row scales; a BF16 blob takes none")
    want = torch.uint8 if fp8 else torch.int16
    if scratch is None:
        scratch = scratch_for(dm)
    if scratch.dtype != want or not scratch.is_contiguous() or scratch.numel() < dm.n * dm.k:
        raise ValueError(f"scratch must be a contiguous {want} buffer of at least {dm.n}x{dm.k} elements")
    w = scratch.reshape(-1)[: dm.n * dm.k].view(dm.n, dm.k)
    dm.dequant(w, dm.k)
    if not fp8:
        return F.linear(x, w.view(torch.bfloat16))
    wb = w.view(torch.float8_e4m3fn).to(torch.bfloat16)
    return (F.linear(x, wb).float() * scale[None, :]).to(torch.bfloat16)
