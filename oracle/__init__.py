"""fp64 CPU oracle of the sparse paged decode step -- test infrastructure only.

Imported by the test suite, the package smoke check and the benchmark's CPU
baseline; never by the library itself.
"""
