"""CPU oracle of the CSA/HCA hybrid attention hot path (test infrastructure).

A plain float64 NumPy model written from the DeepSeek-V4 pages, used only by
``tests/``, the smoke check and the CPU-baseline leg of the benchmark to check
the HIP library.  It shares no code with the library.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, library routines or brute force, except the fidelity of
the whole operator to DeepSeek-V4's unpublished formulas (the pages give none:
the model-card notes list the full Hybrid Attention formulas among what the
documentation does not answer) -- that part is "parity unpinned".
"""
from . import codec, csa  # noqa: F401
