"""Float64 CPU oracle for paged decode attention.

Test infrastructure only: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the library itself.
"""
