"""CPU oracle for the fused dequantize-and-multiply GEMV family.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``gemm_unpack_bit_amd/``): it has its own bit-loop packer, its own
Tile-COO encoder and decoder, and computes every result in float64 from the
logical (unpacked) inputs.

Modules
-------
``formats``    plain bit packing, Tile-COO, codebook-code device tiles (bit loops)
``reference``  float64 y_ref and A = sum_k |x_k w_k| for every variant, plus
               alternative evaluation orders (group identity, Psumbook)
``exact``      exact rational brute force for tiny shapes (fractions.Fraction)
``cref``       a plain C implementation of the uniform GEMV (``cref.c``: its
               own fp16 decoding and bit loop, float64 sums, OpenMP over rows),
               the form timed as the CPU baseline

Acceptance rule used throughout: ``|y - y_ref| <= 2e-3 * A + 1e-6``.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
brute force and the facts the source pages print; no function here is
"parity unpinned".
"""
from . import exact, formats, reference  # noqa: F401

TOL_REL = 2e-3
TOL_ABS = 1e-6
