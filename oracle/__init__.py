"""CPU oracle for the any-precision (bit-plane + LUT) MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The product path (``any_precision_quantized_amd``) never imports it, and this
package imports nothing from the product path: the two share only the seeded
input generators in ``synth``.

Everything here is plain NumPy in float64, slow and written to be checked by
eye against the definitions it cites:

* ``moe``      - bit-plane decode, LUT dequantisation, router, grouping,
                 SwiGLU expert FFN, weighted combine, tolerance magnitudes.
* ``planner``  - the greedy bitwidth planner and a brute-force solver of the
                 budgeted selection problem it approximates.

Parity status: every function is pinned by ``tests/test_oracle.py`` /
``tests/test_planner.py`` (hand-written fixtures, closed forms, brute force and
invariants).  The pages' own measurements (throughput, memory saving, quality)
need trained models and datasets and are not reproduced: parity unpinned for
those, and nothing here claims them.
"""
from . import moe, planner  # noqa: F401
