"""CPU oracle for single-token paged attention decode.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package:
only the tests, the smoke check and the bench's CPU-baseline leg may use it.
It is plain fp64 NumPy that shares no code with the HIP library.
"""
