"""CPU oracle for quantized (INT8 QK / FP8 PV) video-DiT self-attention.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the smoke check
in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
anything from this package.  The HIP library never calls it, and it shares no code,
headers, tables or constants with the HIP path.

The oracle is a plain, slow, FP64 restatement of the numerical program that the pages
"H3 Performance Roadmap" and "Phase 2B Aligned Numerical Prototype" describe, with every
rounding step written out explicitly (``oracle.codecs``).  ``oracle.sattn`` holds the program.

Pins (tests/test_oracle_pins.py, tests/test_codecs.py) tie it to things other than
itself: the textbook softmax attention it must reduce to when rounding is switched
off, the K-mean shift invariance, a grid-exact special case in which every quantizer
is the identity, closed forms (uniform attention), exact scaling invariants, torch's
own float8/bfloat16 codecs and brute force on tiny inputs.

Parity unpinned: none of the pages' own outputs can be reproduced (the Phase 2B
report's SHA-256 needs fixtures that are not published), so byte-parity with the
pages' GB10 kernels is out of reach; every function here is pinned by the properties
above instead.
"""
