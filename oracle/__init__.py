"""CPU oracle for the submanifold convolution: test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.
"""
