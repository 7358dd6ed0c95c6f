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

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle.py``; none is "parity unpinned".  The pages' own NWC v9
bitstream cannot be compared (its format document is not on the pages), so
byte-compatibility with that implementation is a non-goal.
"""
from .nwc_ref import *  # noqa: F401,F403
