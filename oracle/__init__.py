"""CPU oracle for Invariant Bit Packing.

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's
CPU-baseline leg may import anything in this package.  It shares no code with
the HIP library and the product path never imports it.
"""
