"""CPU oracle for the compressed-BF16 batch-1 matvec (NWC-style prefix code).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The product path (``decode_matvec_amd`` and its HIP library) never imports it,
and this package imports nothing from the product: the two share no code.  The
only common dependency is ``synth`` (seeded input generators, no codec
arithmetic).

What it computes follows the "neural-weight-compression 0.9.0" PyPI page
("How it works": byte planes, frequency-ranked unary code with a raw sign bit
and an escape, padding fillers; "Status and limitations": batch-1 path) and the
"Qwen3-4B-NWC-fp8" model card (weight-only fp8 e4m3, per-output-channel scale
applied after the row sum, fp8 bytes entropy-coded and recovered bit for bit).
Where those pages leave a step open, the reading taken is stated at the
function that takes it.

Two writings of the same definitions live here: ``nwc_ref.py`` (pure Python
and numpy, readable, for small inputs) and ``nwc_oracle.c`` with its ctypes
wrapper ``fast.py`` (plain scalar C, for the full-size workloads).  Both write
the same bits (checked).

Pins (CPU tests, ``-m "not gpu"``), what each fixes:
  * hand-derived worked examples (tests/golden/bf16_tiny_codes.txt,
    tests/golden/fp8_tiny_codes.txt): codeword bits, rank order with ties,
    every unary length and an escape, coded sizes -- both writings;
  * Kraft sums in closed form and pairwise prefix-freeness (BF16 and fp8),
    every 16-bit string parsing to its own codeword (BF16);
  * brute-force rank optimality (rearrangement) on small alphabets;
  * closed-form coded size from the histogram = packed stream length;
  * Shannon's bound and the 2 % gate, the pages' entropy figures, a chi-square
    of the generator's exponent histogram against normal-CDF bin masses;
  * lossless round trip of every generated matrix of all five workloads and of
    all 65536 BF16 patterns and all 256 fp8 bytes;
  * exact rational matvec sums on tiny shapes, one-hot/identity special cases,
    the number formats against torch.
No function is left "parity unpinned".  The pages' own NWC v9 bitstream cannot
be compared (its format document is not on the pages), so byte-compatibility
with that implementation is a non-goal.
"""
from .nwc_ref import *  # noqa: F401,F403
