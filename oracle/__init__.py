"""Oracle: a plain, slow CPU reference of the routed MoE layer with IQ4_NL experts.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything under ``oracle/``.  The
product path (``quantized_moe_expert_amd``) never calls it, and this package imports
nothing from the product: the two share no code, no table and no constant.

Floating point is evaluated in float64 (numpy); integer steps (block unpack, top-k
selection, permutation, route sanitisation) are exact.  Every function cites the page
passage it follows; where the pages are silent the plainest reading is taken and named.

Modules:
    iq4nl       -- the IQ4_NL block format: codebook, unpack/dequantise, quantise, pack.
    moe         -- router, top-k selection, gating weights, route sanitisation, permutation,
                   SwiGLU expert, shared expert, weighted combine, the layer and the chain.
    bruteforce  -- a scalar-loop twin of the whole layer for tiny shapes (a pin).

Parity status: every function is pinned by tests in ``tests/test_oracle_*.py``.  Parity
unpinned: the absolute codebook values against real IQ4_NL files (none are available), see
``iq4nl.CODEBOOK``.
"""
from . import iq4nl, moe, bruteforce  # noqa: F401
