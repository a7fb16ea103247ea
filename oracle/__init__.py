"""fp64 CPU oracle for batched speculative-sampling verification.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the benchmark's CPU
baseline, never by the product path.  It shares no code with the HIP library.
"""
