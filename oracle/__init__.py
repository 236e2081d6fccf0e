"""CPU oracle for single-token grouped-query-attention decode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP library and the product path never calls it.

Two independent implementations of the same definition live here:

* ``gqa_oracle.c`` (loaded by :mod:`oracle.ref`): plain C, fp64 loops, its own bf16 and fp8 decoders.
* :mod:`oracle.brute`: pure Python with ``math.fsum``, for tiny inputs.
"""
