"""CPU oracle of the rotated Top-K sparse linear path — test infrastructure.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package. It shares no code with the HIP path and imports
nothing from it.
"""
