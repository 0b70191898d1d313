"""Plain CPU oracle of the sampling chain -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The product path (the HIP library and its binding) never does.
"""
