"""fp64 CPU oracle for exact tiled attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plainly written reference that the HIP kernels are
checked against.  Only the test suite, the smoke check in ``__graft_entry__``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the library under
``exact_tiled_attention_18_amd`` never does, and this package imports nothing
from that library (the two share no code, constants or helpers).

Contents
--------
``attention``        the definition of softmax attention written out in fp64,
                     materialising the full N x N score matrix
                     (``reference``, ``probabilities``, ``online``,
                     ``bruteforce``).
``fp8``              the OCP e4m3 codec written from the format definition,
                     the Sylvester-Hadamard random-sign rotation, per-tile
                     block quantisation, and the attention of the dequantised
                     fp8 operands (the "mirrored" oracle of the fp8 path).

Pins: every function is checked in ``tests/test_oracle_*.py`` against closed
forms, invariants, brute force, hand-derived values (``tests/golden``) and
independent library routines (torch's float64 scaled-dot-product attention,
torch's float8_e4m3fn cast).  No function here is "parity unpinned".
"""
from . import attention, fp8  # noqa: F401
