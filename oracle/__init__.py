"""CPU oracle of the sparse MoE layer -- test infrastructure only.

Only the test suite, the smoke entry point and the benchmark's CPU-baseline leg
may import this package.  The product path never does.
"""
