"""CPU oracle for the NVFP4 block-scaled MoE expert forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table
or constant generator with the HIP implementation under
``nvfp4_block_scaled_04_amd/csrc``; neither side imports the other.

Sources.  The method is described on three web pages of the
``nvfp4-megamoe-kernel`` project: the page titled "CURRENT_BUG.md" (two
renders) and the project's README titled "NVFP4 MegaMoE Kernel".  Each function
cites the README section (or CURRENT_BUG.md section) it follows.  Facts the
pages leave open are stated at the function that needs them, as "reading".

Precision.  Quantisation follows a fixed IEEE fp32 operation sequence (NumPy
float32 arithmetic is correctly rounded); GEMMs, SwiGLU and the combine run in
float64 on exactly decoded operands.

Pinning.  Every function here is pinned by ``tests/test_oracle_*.py`` against
facts that do not come from this package: the pages' rules, the OCP FP8/FP4
format definitions, closed forms, brute force and hand-worked fixtures under
``tests/golden/``.  The quantiser's open decisions are pinned by fixtures that
tell the readings apart: the underflow test after the global scale (blocks
whose raw amax and scaled amax fall on opposite sides of 6 * 2**-9, with
gs = 4 and gs = 0.5), the correctly rounded a_s / 6 and gs / sd (values where
a reciprocal multiply rounds differently and changes a byte), and a
dequantise -> requantise round trip on blocks just above the threshold.  The
near-tie certifier ``quantize.near_ties`` used by the GPU parity tests is
pinned directly (values at, inside and outside the tolerance of a boundary).
"""

from . import formats, quantize, route, layout, moe, mx  # noqa: F401
