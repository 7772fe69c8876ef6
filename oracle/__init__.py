"""CPU oracle of the NOSA decode path (test infrastructure only).

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the library.
"""
